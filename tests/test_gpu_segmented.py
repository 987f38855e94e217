"""GPU parity of the segmented epilogue (one GEMM over concatenated modules,
each keeping its own tensor scale) against the oracle, through every kernel
path: range boundaries inside tiles, empty modules, one-module equality with
the plain GEMM."""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_05_amd as nv
from oracle import nvfp4_ref as ref
from tests.gpu_util import assert_gemm_close, gpu_f32, gpu_u8, host_f32, need_gpu
from workloads import activations, normal_weights

pytestmark = pytest.mark.gpu


def _case(M, rows, K, seed, mults):
    x = activations("t3_outlier1pct", M, K, seed=seed, device="cpu")
    aq = ref.quantize(host_f32(x))
    parts = []
    for i, (r, m) in enumerate(zip(rows, mults)):
        w = normal_weights(r, K, 0.02, seed=seed * 10 + i, device="cpu") * m if r else torch.zeros((0, K))
        parts.append(ref.quantize(w.numpy()) if r else (np.zeros((0, K // 2), np.uint8),
                                                        np.zeros((0, K // 16), np.uint8), np.float32(0.37)))
    wc = np.concatenate([p[0] for p in parts])
    ws = np.concatenate([p[1] for p in parts])
    gs = [p[2] for p in parts]
    return aq, wc, ws, gs


# (M, module rows, K): decode kernel (M <= 64, K % 256 == 0; workgroups of
# 16, 32 and 64 weight rows), generic kernel (K % 128 != 0), streaming kernel
# (>= 256 tiles of 256 x 256); boundaries fall inside workgroup tiles, one
# module is empty.  The fused GDN in-projection (8192 | 4096 | 48 | 48 rows,
# K = 5120) at 1 and 64 rows is the decode step the bench times.
SHAPES = [
    (5, (40, 0, 17, 7), 512),
    (3, (8192, 4096, 48, 48), 512),
    (1, (8192, 4096, 48, 48), 5120),
    (64, (8192, 4096, 48, 48), 5120),
    (20, (2000, 3000, 120), 256),
    (64, (8192 // 64, 48, 48, 300), 1024),
    (37, (100, 3, 60), 144),
    (300, (130, 0, 77, 49), 384),
    (4096, (2048, 48, 48, 2000), 256),
    (4130, (3000, 1, 1190), 512),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_segmented_matches_oracle(shape):
    need_gpu()
    M, rows, K = shape
    print(f"[segmented] M={M} module rows={rows} K={K}", flush=True)
    mults = [1.0, 9.0, 0.07, 3.0][:len(rows)]
    aq, wc, ws, gs = _case(M, rows, K, seed=len(rows) + K, mults=mults)
    Y, S = ref.gemm_segmented_ref(*aq, wc, ws, gs, rows)
    gs_dev = torch.tensor([float(g) for g in gs], dtype=torch.float32, device="cuda")
    for dt in (torch.float32, torch.bfloat16):
        y = nv.gemm_segmented(gpu_u8(aq[0]), gpu_u8(aq[1]), gpu_f32(aq[2]), gpu_u8(wc), gpu_u8(ws), gs_dev, rows,
                              out_dtype=dt)
        torch.cuda.synchronize()
        assert_gemm_close(y, Y, S, f"segmented {shape} {dt}")


@pytest.mark.parametrize("shape", [(3, 200, 512), (300, 700, 384), (4096, 4096, 256)])
def test_one_module_is_the_plain_gemm(shape):
    """Same kernels: a one-module segmented GEMM is bit-identical to nvfp4_gemm."""
    need_gpu()
    M, N, K = shape
    x = activations("t3_outlier1pct", M, K, seed=5, device="cuda")
    w = normal_weights(N, K, 0.02, seed=6, device="cuda")
    a = nv.quantize(x)
    b = nv.quantize(w)
    y0 = nv.gemm(*a, *b, out_dtype=torch.bfloat16)
    y1 = nv.gemm_segmented(*a, b[0], b[1], b[2].reshape(1), [N], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
