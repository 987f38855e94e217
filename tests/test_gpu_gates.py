"""GDN gate epilogue (nvfp4_gemm_segmented_gates) against the oracle.

Columns outside the two gate modules must be bit-identical to
nvfp4_gemm_segmented.  A gate column must lie within the GEMM bound carried
through the gate, |y - G| <= |dG/dv| 1e-4 Sabs with |dG/dv| <= exp(A_log) for
the decay gate and 1/4 for sigmoid, plus the fp32 evaluation (the sum
v + dt_bias rounded, a few ulp of the functions) and, for bf16 output, half
a bf16 ulp.  Shapes run through all three GEMM kernels (decode, generic and
streaming) with gate ranges that cross wave and tile boundaries."""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_05_amd as nv
from oracle import nvfp4_ref as ref
from tests.gpu_util import (GEMM_RTOL, assert_codes_equal, assert_gemm_close, gpu_u8, host_f32, need_gpu,
                            oracle_quantize_host)
from workloads import activations, normal_weights

pytestmark = pytest.mark.gpu


def gate_params(n, seed):
    """Synthetic per-head A_log and dt_bias: A = U(1, 16), so A_log = log A, and
    dt_bias the inverse softplus of dt = exp(U(log 1e-3, log 1e-1))."""
    rng = np.random.default_rng(seed)
    a_log = np.log(rng.uniform(1.0, 16.0, n)).astype(np.float32)
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), n))
    dt_bias = (dt + np.log(-np.expm1(-dt))).astype(np.float32)
    return a_log, dt_bias


def _case(M, K, rows, decay, write, seed, rows_sample=None):
    dev = need_gpu()
    x = activations("t3_outlier1pct", M, K, seed=seed, device=dev)
    a = nv.quantize(x)
    # weights quantized by the oracle on the host (the GPU quantizer is pinned elsewhere)
    omods = [oracle_quantize_host(normal_weights(r, K, 0.02, seed=seed * 10 + i, device="cpu"))
             for i, r in enumerate(rows)]
    ow_c = np.concatenate([m[0] for m in omods])
    ow_s = np.concatenate([m[1] for m in omods])
    ow_g = np.array([m[2] for m in omods], dtype=np.float32)
    wc, wsc = gpu_u8(ow_c), gpu_u8(ow_s)
    mgs = torch.from_numpy(ow_g).to(dev)
    n_dec = rows[decay] if decay >= 0 else 1
    a_log, dt_bias = gate_params(n_dec, seed)
    gpu = dict(decay_module=decay, a_log=torch.from_numpy(a_log).to(dev) if decay >= 0 else None,
               dt_bias=torch.from_numpy(dt_bias).to(dev) if decay >= 0 else None, write_module=write)
    starts = np.concatenate([[0], np.cumsum(rows)])
    gate_cols = np.zeros(starts[-1], bool)
    for m in (decay, write):
        if m >= 0:
            gate_cols[starts[m]:starts[m + 1]] = True
    sample = np.arange(M) if rows_sample is None else rows_sample
    sample_t = torch.from_numpy(sample).to(dev)
    # activations: the oracle's quantization of the sampled rows with the
    # oracle's tensor scale of the whole tensor, equal to the GPU's bytes
    xh = host_f32(x)
    ah = ref.quantize(xh[sample], g=ref.global_scale(xh))
    assert float(a[2].item()) == float(ah[2])
    assert_codes_equal(a[0][sample_t], a[1][sample_t], ah[0], ah[1], "activations")
    del xh
    G, Y, S = ref.gemm_segmented_gates_ref(*ah, ow_c, ow_s, ow_g, rows, decay, a_log, dt_bias, write)
    for od in (torch.float32, torch.bfloat16):
        y = nv.gemm_segmented_gates(*a, wc, wsc, mgs, rows, out_dtype=od, **gpu)
        y0 = nv.gemm_segmented(*a, wc, wsc, mgs, rows, out_dtype=od)
        torch.cuda.synchronize()
        assert torch.equal(y[:, ~torch.from_numpy(gate_cols).to(dev)], y0[:, ~torch.from_numpy(gate_cols).to(dev)]), \
            f"non-gate columns differ from nvfp4_gemm_segmented ({od})"
        # the segmented epilogue itself, on the columns without a gate
        assert_gemm_close(y0[sample_t][:, torch.from_numpy(~gate_cols).to(dev)], Y[:, ~gate_cols], S[:, ~gate_cols],
                          f"segmented epilogue ({od})")
        yv = host_f32(y[sample_t]).astype(np.float64)
        del y0
        tol = np.zeros_like(G)
        if decay >= 0:
            sl = slice(starts[decay], starts[decay + 1])
            ea = np.exp(a_log.astype(np.float64))
            tol[:, sl] = ea * (GEMM_RTOL * S[:, sl] + np.abs(Y[:, sl] + dt_bias) * 2.0 ** -22) + \
                2.0 ** -20 * np.abs(G[:, sl])
        if write >= 0:
            sl = slice(starts[write], starts[write + 1])
            tol[:, sl] = 0.25 * GEMM_RTOL * S[:, sl] + 2.0 ** -20 * np.abs(G[:, sl])
        if od == torch.bfloat16:
            tol = tol + 2.0 ** -8 * (np.abs(G) + tol)
        err = np.abs(yv - G)[:, gate_cols]
        t = tol[:, gate_cols]
        bad = np.argwhere(err > t)
        assert bad.size == 0, (f"{od}: {len(bad)} gate values out of tolerance, first {bad[:3].tolist()}: "
                               f"y={yv[:, gate_cols][tuple(bad[0])]!r} G={G[:, gate_cols][tuple(bad[0])]!r}")


@pytest.mark.parametrize("M", [1, 7, 20, 40])
@pytest.mark.parametrize("rows", [(120, 48, 48, 40), (256, 128, 48, 48)])
def test_gates_decode_kernel(M, rows):
    print(f"[gates] decode M={M} rows={rows}", flush=True)
    _case(M, 512, list(rows), 1 if rows[0] == 120 else 2, 2 if rows[0] == 120 else 3, seed=M + rows[0])


def test_gates_generic_kernel_and_module_order():
    print("[gates] generic K=400, decay module first, write module last", flush=True)
    _case(97, 400, [48, 200, 48], 0, 2, seed=3)
    print("[gates] generic, write gate only", flush=True)
    _case(97, 400, [48, 200, 48], -1, 0, seed=4)


def test_gates_streaming_kernel_across_tile_boundaries():
    # N = 4168: a covers columns 4070..4117 (crossing the 4096 tile and wave
    # boundary), b 4118..4165; M = 4096 gives 16 x 17 big tiles
    print("[gates] streaming M=4096 rows=(4070, 48, 48, 2) K=1024", flush=True)
    _case(4096, 1024, [4070, 48, 48, 2], 1, 2, seed=5, rows_sample=np.array([0, 1, 255, 256, 1777, 4095]))


def test_gates_fused_gdn_in_projection():
    # the fused GDN in-projection (qkv 8192 | z 4096 | a 48 | b 48) at 4096 tokens
    print("[gates] fused GDN in-projection 4096 x 12384 x 5120", flush=True)
    _case(4096, 5120, [8192, 4096, 48, 48], 2, 3, seed=6, rows_sample=np.array([0, 513, 2048, 4095]))


def test_gates_fused_gdn_in_projection_32k_tokens():
    # the same projection at 32768 tokens with bf16 and fp32 output: the
    # launch the bench times (128 x 49 big tiles)
    print("[gates] fused GDN in-projection 32768 x 12384 x 5120", flush=True)
    _case(32768, 5120, [8192, 4096, 48, 48], 2, 3, seed=8,
          rows_sample=np.array([0, 255, 256, 16383, 20000, 32767]))
