"""nvfp4_gemm_swiglu_quantize: the gate/up GEMM with SwiGLU and NVFP4
quantization in its epilogue.

Two checks per shape:
  * h (fp32, written on request) against the fp64 oracle: the GEMM bound
    |v - Y| <= 1e-4 Sabs for gate and up, carried through h = silu(g) u
    (|silu'| <= 1.1, |d h / d u| = |silu(g)|), plus a few fp32 ulp and
    |g| 2^-22 relative (the hardware exp2 of g log2 e);
  * the codes and scales bit-identical to the oracle's quantization of that
    h (every row; h is the kernel's own fp32 output, so both sides quantize
    the same values) with the same tensor scale, and to nvfp4_quantize of h."""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_05_amd as nv
from oracle import nvfp4_ref as ref
from tests.gpu_util import (GEMM_RTOL, assert_codes_equal, assert_quantize_matches_oracle_full, host_f32, need_gpu,
                            oracle_quantize_host, to_gpu_quantized)
from workloads import activations, normal_weights

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,F,K,sample", [(300, 192, 256, None), (257, 64, 128, None), (1000, 512, 1024, None),
                                          (4096, 17408, 5120, (0, 1, 255, 2049, 4095)),
                                          (32768, 17408, 5120, (0, 255, 256, 16383, 32767))])
def test_swiglu_quantize_epilogue(M, F, K, sample):
    # the last shape is the MLP of a 32768-token layer, the launch the bench times
    dev = need_gpu()
    print(f"[swiglu] M={M} F={F} K={K}", flush=True)
    x = activations("t3_outlier1pct", M, K, seed=M + F, device=dev)
    a = nv.quantize(x)
    xh = host_f32(x)
    g_a = ref.global_scale(xh)
    assert float(a[2].item()) == float(g_a)
    assert_quantize_matches_oracle_full(x, a[0], a[1], g_a, "activations")
    ow = oracle_quantize_host(normal_weights(2 * F, K, 0.015, seed=F, device="cpu"))   # weights from the oracle
    w = to_gpu_quantized(ow)
    h = torch.full((M, F + 8), float("nan"), dtype=torch.float32, device=dev)     # ldh > F
    nv.gemm_swiglu_quantize(*a, *w, torch.ones(1, device=dev), h=h)               # h for calibration
    hg = nv.quantize(h[:, :F].contiguous())[2].clone()                            # amax / 2688
    codes, scales, _ = nv.gemm_swiglu_quantize(*a, *w, hg, h=h)
    codes_only = nv.gemm_swiglu_quantize(*a, *w, hg)                               # no h: the chain's form
    torch.cuda.synchronize()
    assert torch.equal(codes_only[0], codes) and torch.equal(codes_only[1], scales), "codes depend on h"
    del codes_only
    assert torch.isnan(h[:, F:]).all(), "h written past column F"
    hv = h[:, :F].contiguous()
    del h
    assert float(hg.item()) == float(ref.global_scale(host_f32(hv))), "h tensor scale"
    n = assert_quantize_matches_oracle_full(hv, codes, scales, np.float32(hg.item()), "fused vs oracle quantize of h")
    print(f"  all {n} code and scale bytes of h match the oracle", flush=True)
    c2, s2, _ = nv.quantize(hv, hg, from_amax=False)
    torch.cuda.synchronize()
    assert_codes_equal(codes, scales, c2.cpu().numpy(), s2.cpu().numpy(), "fused vs nvfp4_quantize of h")
    rows = np.arange(M) if sample is None else np.array(sample)
    rows_t = torch.from_numpy(rows).to(dev)
    ah = ref.quantize(xh[rows], g=g_a)            # the oracle's activations (equal to the GPU's, checked above)
    del xh
    H, G, U, SG, SU = ref.gemm_swiglu_ref(*ah, *ow)
    eg, eu = GEMM_RTOL * SG, GEMM_RTOL * SU
    # plus the fp32 evaluation: a few ulp, and |g| 2^-23 relative from the exp2 argument's rounding
    tol = 1.1 * (np.abs(U) + eu) * eg + (np.abs(ref.silu(G)) + 1.1 * eg) * eu + \
        (2.0 ** -20 + np.abs(G) * 2.0 ** -22) * np.abs(H) + 1e-30
    err = np.abs(host_f32(hv[rows_t]).astype(np.float64) - H)
    bad = np.argwhere(err > tol)
    assert bad.size == 0, f"{len(bad)} h values out of tolerance, first {bad[:3].tolist()}"
