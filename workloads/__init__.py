"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This package draws random numbers and nothing else: it contains none of the
NVFP4 arithmetic (no scales, no rounding, no codes).  Both the CPU oracle and
the HIP path consume what it returns.
"""
from .generators import (  # noqa: F401
    CONFIGS,
    ProjectionSpec,
    activations,
    normal_weights,
    stats,
)
