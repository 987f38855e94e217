"""Helpers for the GPU parity tests: device transfer and the tolerance checks.

The expected values always come from ``oracle/`` (run here on the host) or
from the hand-worked fixtures; GPU results are only ever compared, never fed
back into the oracle.
"""
import numpy as np
import pytest
import torch

from oracle import nvfp4_ref as ref

GEMM_RTOL = 1e-4  # |y - Y| <= 1e-4 * sum_k |a_k w_k| per element


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return torch.device("cuda:0")


def gpu_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def gpu_f32(v):
    return torch.tensor([float(v)], dtype=torch.float32).cuda()


def host_f32(x: torch.Tensor) -> np.ndarray:
    """Values of a (bf16 or fp32) tensor as fp32 numpy, exactly."""
    return x.detach().float().cpu().numpy()


def assert_codes_equal(got_codes, got_scales, want_codes, want_scales, what=""):
    gc = got_codes.cpu().numpy() if isinstance(got_codes, torch.Tensor) else got_codes
    gs = got_scales.cpu().numpy() if isinstance(got_scales, torch.Tensor) else got_scales
    bad_s = np.argwhere(gs != want_scales)
    assert bad_s.size == 0, f"{what}: {len(bad_s)} scale mismatches, first at {bad_s[:3].tolist()}: " \
                            f"got {gs[tuple(bad_s[0])]:#x} want {want_scales[tuple(bad_s[0])]:#x}"
    bad_c = np.argwhere(gc != want_codes)
    assert bad_c.size == 0, f"{what}: {len(bad_c)} code-byte mismatches, first at {bad_c[:3].tolist()}: " \
                            f"got {gc[tuple(bad_c[0])]:#04x} want {want_codes[tuple(bad_c[0])]:#04x}"


def assert_gemm_close(y: torch.Tensor, Y: np.ndarray, Sabs: np.ndarray, what=""):
    """fp32 output: |y - Y| <= 1e-4 Sabs.  bf16 output adds the bf16 rounding
    of the fp32 result, at most half a bf16 ulp: 2^-8 of its magnitude."""
    yv = y.float().cpu().numpy().astype(np.float64)
    tol = GEMM_RTOL * Sabs
    if y.dtype == torch.bfloat16:
        tol = tol + 2.0 ** -8 * (np.abs(Y) + tol)
    err = np.abs(yv - Y)
    bad = np.argwhere(err > tol)
    assert bad.size == 0, (f"{what}: {len(bad)} elements out of tolerance, first {bad[:3].tolist()}: "
                           f"y={yv[tuple(bad[0])]!r} Y={Y[tuple(bad[0])]!r} Sabs={Sabs[tuple(bad[0])]!r}")
    return float(np.max(err / np.maximum(Sabs, 1e-300)))


def oracle_quantize(x: torch.Tensor, g=None):
    return ref.quantize(host_f32(x), g=g)
