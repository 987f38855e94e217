"""MI355X-native NVFP4 W4A4 linear layer: quantize, GEMM, fused-scale harmonize.

The computation lives in ``libnvfp4.so`` (hand-written HIP for gfx950 behind
the C ABI of ``include/nvfp4.h``); this package is its thin Python binding.
"""
from ._lib import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    Nvfp4Error,
    gemm,
    gemm_segmented,
    gemm_segmented_gates,
    gemm_swiglu_quantize,
    gdn_recurrence,
    harmonize_fused_scales,
    load,
    quantize,
    quantize_gemm,
    quantize_gemm_no_alloc,
)
