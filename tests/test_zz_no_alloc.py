"""nvfp4_quantize_gemm_no_alloc, the entry point for callers that cannot
allocate (its quantized activations live in a static device array), against
nvfp4_quantize_gemm with a caller workspace: bit-identical outputs on two
calls in a row, the second one smaller, and both within the GEMM bound of
the fp64 oracle.  Weights, activation codes and the calibrated tensor scale
come from the oracle on the host."""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_05_amd as nv
from oracle import nvfp4_ref as ref
from tests.gpu_util import assert_gemm_close, gpu_f32, gpu_u8, host_f32, need_gpu
from workloads import activations, normal_weights

pytestmark = pytest.mark.gpu

# (M, N, K, activation dtype, output dtype): both take the scratch (M > 2,
# or fp32 activations); the second call is the smaller one
CASES = [(300, 1024, 2048, torch.bfloat16, torch.float32),
         (40, 512, 1024, torch.float32, torch.bfloat16)]


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def test_no_alloc_matches_the_workspace_entry_point_on_two_calls():
    dev = need_gpu()
    lib = nv.load()
    for i, (M, N, K, xdt, odt) in enumerate(CASES):
        print(f"[no alloc] call {i + 1}: M={M} N={N} K={K} x {xdt} out {odt}", flush=True)
        x = activations("t3_outlier1pct", M, K, seed=50 + i, device="cpu", dtype=xdt)
        xh = host_f32(x)
        g = ref.global_scale(xh)                                  # calibrated static scale
        ow = ref.quantize(normal_weights(N, K, 0.02, seed=60 + i, device="cpu").numpy())
        w = (gpu_u8(ow[0]), gpu_u8(ow[1]), gpu_f32(ow[2]))
        xd, gd = x.to(dev), gpu_f32(g)
        in_dt = 1 if xdt == torch.bfloat16 else 0
        out_dt = 1 if odt == torch.bfloat16 else 0
        need = lib.nvfp4_quantize_gemm_workspace_size(M, N, K, in_dt, out_dt)
        assert 0 < need <= lib.nvfp4_quantize_gemm_no_alloc_max_bytes()
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        y_ws = nv.quantize_gemm(xd, gd, *w, out_dtype=odt, workspace=ws)
        y_na = torch.full((M, N), float("nan"), dtype=odt, device=dev)
        nv.quantize_gemm_no_alloc(xd, gd, *w, out_dtype=odt, out=y_na)
        torch.cuda.synchronize()
        assert torch.equal(_bits(y_na), _bits(y_ws)), f"call {i + 1}: outputs differ from nvfp4_quantize_gemm"
        Y, S = ref.gemm_ref(*ref.quantize(xh, g=g), *ow)
        r = assert_gemm_close(y_na, Y, S, f"no-alloc call {i + 1}")
        print(f"  bit-identical to the workspace call; max |err|/sum|a w| = {r:.2e}", flush=True)
