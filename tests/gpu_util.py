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


def oracle_threads():
    """Host threads for the oracle over big tensors (numpy releases the GIL in
    its array loops): the host's share, at most 16."""
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def assert_quantize_matches_oracle_full(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, g,
                                        what="", chunk_rows=512):
    """Every code byte and scale byte of a GPU-quantized tensor against
    ``ref.quantize`` of the same values with the same tensor scale g (the
    quantizer is row-independent once g is fixed), in row chunks on host
    threads.  x is the GPU input (bf16 or fp32); codes and scales are the GPU
    results; g is the oracle's tensor scale (np.float32)."""
    from concurrent.futures import ThreadPoolExecutor

    rows = x.shape[0]
    xh = x.detach().cpu()                                   # exact bf16 / fp32 values
    ch, sh = codes.cpu().numpy(), scales.cpu().numpy()
    g = np.float32(g)

    def check(r0):
        r1 = min(rows, r0 + chunk_rows)
        oc, os_, _ = ref.quantize(xh[r0:r1].float().numpy(), g=g)
        bad_s = np.argwhere(sh[r0:r1] != os_)
        bad_c = np.argwhere(ch[r0:r1] != oc)
        first = None
        if bad_s.size:
            i = tuple(bad_s[0])
            first = f"scale [{r0 + i[0]}, {i[1]}] got {sh[r0 + i[0], i[1]]:#x} want {os_[i]:#x}"
        elif bad_c.size:
            i = tuple(bad_c[0])
            first = f"code byte [{r0 + i[0]}, {i[1]}] got {ch[r0 + i[0], i[1]]:#04x} want {oc[i]:#04x}"
        return len(bad_s), len(bad_c), first

    with ThreadPoolExecutor(oracle_threads()) as ex:
        res = list(ex.map(check, range(0, rows, chunk_rows)))
    n_s = sum(r[0] for r in res)
    n_c = sum(r[1] for r in res)
    firsts = [r[2] for r in res if r[2]]
    assert n_s == 0 and n_c == 0, f"{what}: {n_s} scale and {n_c} code-byte mismatches; first: {firsts[:1]}"
    return codes.numel() + scales.numel()


def oracle_quantize_host(x, g=None, chunk_rows=512):
    """ref.quantize of a host tensor (numpy or CPU torch, any float dtype),
    in row chunks on host threads; g = None takes the tensor scale of the
    whole tensor (ref.global_scale).  Same bytes as ref.quantize(x, g)."""
    from concurrent.futures import ThreadPoolExecutor

    if isinstance(x, torch.Tensor):
        x = x.detach().float().cpu().numpy()
    x = np.asarray(x, dtype=np.float32)
    g = ref.global_scale(x) if g is None else np.float32(g)
    rows = x.shape[0]
    with ThreadPoolExecutor(oracle_threads()) as ex:
        parts = list(ex.map(lambda r0: ref.quantize(x[r0:r0 + chunk_rows], g=g), range(0, rows, chunk_rows)))
    if not parts:
        return ref.quantize(x, g=g)
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]), g


def to_gpu_quantized(q):
    """(codes, scales, g) from the host oracle, as device tensors."""
    return gpu_u8(q[0]), gpu_u8(q[1]), gpu_f32(q[2])
