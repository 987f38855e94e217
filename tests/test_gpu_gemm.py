"""GPU GEMM parity: outputs within |y - Y| <= 1e-4 * sum_k |a_k w_k| of the
fp64 oracle; the in-kernel dequantization bit-exact through an identity weight."""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_05_amd as nv
from oracle import nvfp4_ref as ref
from tests.gpu_util import assert_gemm_close, gpu_f32, gpu_u8, host_f32, need_gpu
from workloads import CONFIGS, activations, normal_weights

pytestmark = pytest.mark.gpu


def _run(aq, wq, out_dtype=torch.float32, k=None):
    (ac, as_, ga), (wc, ws, gw) = aq, wq
    y = nv.gemm(gpu_u8(ac), gpu_u8(as_), gpu_f32(ga), gpu_u8(wc), gpu_u8(ws), gpu_f32(gw),
                out_dtype=out_dtype, k=k)
    torch.cuda.synchronize()
    return y


def _selection_weight(N, K):
    """W [N, K] with one code 2 (= 1.0) per row, at column n % K, every block
    scale 0x38 (= 1.0) and g_w = 1: y[m, n] = deq(A)[m, n % K] exactly, since
    each output is a single product."""
    codes = np.zeros((N, K), np.uint8)
    codes[np.arange(N), np.arange(N) % K] = 2
    return ref.pack_codes(codes), np.full((N, K // 16), 0x38, np.uint8), np.float32(1)


def _all_code_scale_pairs(M, K):
    """A [M, K] whose blocks run through every E4M3 scale byte 0x00..0x7E
    (subnormals and 0 included) and hold all 16 E2M1 codes each, rotated per
    row, so every (code, scale) pair occurs many times."""
    nb = K // 16
    codes = (np.arange(K)[None, :] + np.arange(M)[:, None]) % 16
    scales = (np.arange(M)[:, None] * nb + np.arange(nb)[None, :]) % 127
    return ref.pack_codes(codes.astype(np.uint8)), scales.astype(np.uint8), np.float32(1)


def _assert_selected_exactly(y, aq, N, K, what):
    """y[m, n] == deq(A)[m, n % K] bit for bit.  A zero output is +0: the
    accumulator starts at +0, and the sum of +0 and the -0 product of a
    negative zero code is +0 under round-to-nearest-even."""
    deq = ref.dequantize(aq[0], aq[1], 1.0)
    want = (deq[:, np.arange(N) % K] + 0.0).astype(np.float32)          # -0 -> +0
    got = y.float().cpu().numpy()
    bad = np.argwhere(got.view(np.uint32) != want.view(np.uint32))
    assert bad.size == 0, (f"{what}: {len(bad)} outputs differ from the exact dequantized value, first "
                           f"{bad[:3].tolist()}: got {got[tuple(bad[0])]!r} want {want[tuple(bad[0])]!r}")


def test_identity_weight_dequantizes_every_code_and_scale_exactly():
    """W = I (code 2 = 1.0, scale 1.0, g_w = 1) and g_a = 1: every output is a
    single product, so y = deq(A) bit for bit, over all 16 codes x 127 scales.
    M = 127 and one 256-wide tile: the generic kernel."""
    need_gpu()
    K = 256
    codes = np.tile(np.arange(16, dtype=np.uint8), (127, K // 16))      # [127, K] one code per value
    scales = np.repeat(np.arange(127, dtype=np.uint8)[:, None], K // 16, axis=1)
    ac = ref.pack_codes(codes)
    for dt in (torch.float32, torch.bfloat16):
        y = _run((ac, scales, np.float32(1)), _selection_weight(K, K), out_dtype=dt)
        _assert_selected_exactly(y, (ac, scales), K, K, f"generic kernel {dt}")


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_exact_dequant_through_streaming_kernel(dt):
    """M = N = 4096, K = 256: 256 output tiles of 256 x 256 with K % 128 == 0
    and aligned operands, the shape class of the large-tile streaming kernel
    (the bench's prefill GEMMs); every (code, scale) pair, bit for bit."""
    need_gpu()
    M = N = 4096
    K = 256
    aq = _all_code_scale_pairs(M, K)
    y = _run(aq, _selection_weight(N, K), out_dtype=dt)
    _assert_selected_exactly(y, aq, N, K, f"streaming kernel {dt}")


@pytest.mark.parametrize("m", [1, 16, 64])
def test_exact_dequant_through_decode_kernel(m):
    """M <= 64 with K % 256 == 0: the decode kernel; K = 4096 gives 256
    blocks per row, so even one row runs through all 127 scales and every
    block holds all 16 codes; bit for bit, fp32 and bf16 output."""
    need_gpu()
    N, K = 4096, 4096
    aq = _all_code_scale_pairs(m, K)
    wq = _selection_weight(N, K)
    for dt in (torch.float32, torch.bfloat16):
        y = _run(aq, wq, out_dtype=dt)
        _assert_selected_exactly(y, aq, N, K, f"decode kernel M={m} {dt}")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_tiny_config(out_dtype):
    need_gpu()
    cfg = CONFIGS["tiny"]
    kind, rows, cols, dtype = cfg["x"]
    x = activations(kind, rows, cols, seed=cfg["seed"], device="cpu", dtype=dtype)
    p = cfg["projections"][0]
    w = normal_weights(p.n, p.k, p.std, seed=cfg["seed"] * 100, device="cpu")
    aq, wq = ref.quantize(host_f32(x)), ref.quantize(w.numpy())
    Y, S = ref.gemm_ref(*aq, *wq)
    y = _run(aq, wq, out_dtype)
    assert_gemm_close(y, Y, S, f"tiny {out_dtype}")


@pytest.mark.parametrize("m", [1, 8, 32, 64])
def test_decode_config(m):
    need_gpu()
    cfg = CONFIGS["decode"]
    kind, _, cols, dtype = cfg["x"]
    p = cfg["projections"][0]
    print(f"[gemm parity] decode M={m} N={p.n} K={p.k}", flush=True)
    x = activations(kind, m, cols, seed=cfg["seed"], device="cpu", dtype=dtype)
    w = normal_weights(p.n, p.k, p.std, seed=cfg["seed"] * 100, device="cpu")
    aq, wq = ref.quantize(host_f32(x)), ref.quantize(w.numpy())
    Y, S = ref.gemm_ref(*aq, *wq)
    y = _run(aq, wq)
    assert_gemm_close(y, Y, S, f"decode M={m}")


@pytest.mark.parametrize("shape", [(37, 100, 48), (5, 48, 16), (130, 257, 144), (64, 300, 256),
                                   (1, 7, 4096), (300, 129, 384), (513, 520, 1040)])
def test_ragged_shapes(shape):
    """Tails in M, N and K (K % 128 != 0 takes the generic loader)."""
    need_gpu()
    M, N, K = shape
    print(f"[gemm parity] ragged M={M} N={N} K={K}", flush=True)
    x = activations("t3_outlier1pct", M, K, seed=M + N + K, device="cpu")
    w = normal_weights(N, K, 0.02, seed=M * N, device="cpu")
    aq, wq = ref.quantize(host_f32(x)), ref.quantize(w.numpy())
    Y, S = ref.gemm_ref(*aq, *wq)
    for dt in (torch.float32, torch.bfloat16):
        y = _run(aq, wq, dt)
        assert_gemm_close(y, Y, S, f"ragged {shape} {dt}")


@pytest.mark.parametrize("shape", [(4113, 4140, 1024), (4096, 4096, 256), (3000, 6000, 640)])
def test_large_tile_kernel_with_ragged_edges(shape):
    """Shapes large enough for the 256x256 streaming kernel, with M and N tails."""
    need_gpu()
    M, N, K = shape
    print(f"[gemm parity] streaming kernel M={M} N={N} K={K}", flush=True)
    x = activations("t3_outlier1pct", M, K, seed=7, device="cpu")
    w = normal_weights(N, K, 0.02, seed=8, device="cpu")
    aq, wq = ref.quantize(host_f32(x)), ref.quantize(w.numpy())
    Y, S = ref.gemm_ref(*aq, *wq)
    for dt in (torch.float32, torch.bfloat16):
        y = _run(aq, wq, dt)
        assert_gemm_close(y, Y, S, f"large {shape} {dt}")


@pytest.mark.parametrize("shape", [(64, 100, 17408), (3, 49, 17408), (20, 96, 768), (33, 48, 2560),
                                   (16, 12288, 4096), (8, 5120, 1024), (2, 12384, 512), (40, 12400, 256),
                                   (48, 1000, 1280), (49, 640, 512)])
def test_decode_kernel_k_splits(shape):
    """M <= 64 with K % 256 == 0 takes the decode kernel: K quarters of 0..17
    tiles, full and partial refill rounds, scale runs above 64 KiB of LDS, and
    1, 2, 3 and 4 weight blocks of 16 rows per workgroup (N = 100, 5120,
    12288, 12384)."""
    need_gpu()
    M, N, K = shape
    print(f"[gemm parity] decode kernel M={M} N={N} K={K}", flush=True)
    x = activations("t3_outlier1pct", M, K, seed=M + K, device="cpu")
    w = normal_weights(N, K, 0.02, seed=N + K, device="cpu")
    aq, wq = ref.quantize(host_f32(x)), ref.quantize(w.numpy())
    Y, S = ref.gemm_ref(*aq, *wq)
    for dt in (torch.float32, torch.bfloat16):
        y = _run(aq, wq, dt)
        assert_gemm_close(y, Y, S, f"decode {shape} {dt}")


def test_unaligned_operand_pointers_take_generic_path():
    need_gpu()
    M, N, K = 40, 72, 256
    x = activations("t3_outlier1pct", M, K, seed=1, device="cpu")
    w = normal_weights(N, K, 0.02, seed=2, device="cpu")
    (ac, as_, ga), (wc, ws, gw) = ref.quantize(host_f32(x)), ref.quantize(w.numpy())
    Y, S = ref.gemm_ref(ac, as_, ga, wc, ws, gw)
    # place the codes at an odd byte offset inside a larger buffer
    buf = torch.zeros(ac.size + 1, dtype=torch.uint8, device="cuda")
    buf[1:] = gpu_u8(ac).flatten()
    a_view = buf[1:].view(M, K // 2)
    y = nv.gemm(a_view, gpu_u8(as_), gpu_f32(ga), gpu_u8(wc), gpu_u8(ws), gpu_f32(gw))
    torch.cuda.synchronize()
    assert_gemm_close(y, Y, S, "unaligned A codes")


def test_output_row_stride():
    need_gpu()
    M, N, K = 64, 96, 256
    x = activations("t3_outlier1pct", M, K, seed=3, device="cpu")
    w = normal_weights(N, K, 0.02, seed=4, device="cpu")
    aq, wq = ref.quantize(host_f32(x)), ref.quantize(w.numpy())
    Y, S = ref.gemm_ref(*aq, *wq)
    big = torch.full((M, 128), 7.0, device="cuda")
    out = big[:, :N]
    (ac, as_, ga), (wc, ws, gw) = aq, wq
    nv.gemm(gpu_u8(ac), gpu_u8(as_), gpu_f32(ga), gpu_u8(wc), gpu_u8(ws), gpu_f32(gw), out=out)
    torch.cuda.synchronize()
    assert_gemm_close(out, Y, S, "ldy > N")
    assert torch.all(big[:, N:] == 7.0)


def test_deterministic_repeat():
    need_gpu()
    M, N, K = 512, 768, 1024
    x = activations("t3_outlier1pct", M, K, seed=8, device="cuda")
    w = normal_weights(N, K, 0.02, seed=9, device="cuda")
    a = nv.quantize(x)
    b = nv.quantize(w)
    y1 = nv.gemm(*a, *b)
    y2 = nv.gemm(*a, *b)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_operands_past_2gib_take_64bit_offsets():
    """A [262181 x 16384]: 4.3 G values (past 2^32 elements in the quantizer)
    and 2.15 GB of codes (past 2^31 bytes, so the GEMM takes the generic
    kernel, whose offsets are 64-bit).  The tensor scale is given, so sampled
    rows on both sides of the 2 GiB mark can be checked against the oracle."""
    dev = need_gpu()
    M, N, K = 262181, 200, 16384
    assert M * (K // 2) > 2 ** 31 and M * K > 2 ** 32
    print(f"[gemm] past 2 GiB: A {M}x{K} bf16, W {N}x{K}", flush=True)
    gen = torch.Generator(device=dev).manual_seed(77)
    x = torch.randn((M, K), generator=gen, device=dev, dtype=torch.bfloat16)
    g = np.float32(0.0025)
    a = nv.quantize(x, torch.tensor([g], device=dev), from_amax=False)
    w = normal_weights(N, K, 0.02, seed=78, device=dev)
    b = nv.quantize(w)
    y = nv.gemm(*a, *b, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = np.array([0, 131071, 262143, 262144, 262145, M - 1])   # 262144 * 8192 = 2^31
    rows_t = torch.from_numpy(rows).to(dev)
    oa = ref.quantize(host_f32(x[rows_t]), g=g)
    assert np.array_equal(a[0][rows_t].cpu().numpy(), oa[0]) and np.array_equal(a[1][rows_t].cpu().numpy(), oa[1])
    ow = ref.quantize(host_f32(w))
    assert np.array_equal(b[0].cpu().numpy(), ow[0]) and np.array_equal(b[1].cpu().numpy(), ow[1])
    assert float(b[2].item()) == float(ow[2])
    Y, S = ref.gemm_ref(*oa, *ow)
    assert_gemm_close(y[rows_t], Y, S, "A past 2 GiB")


def test_streaming_and_decode_kernels_just_below_their_offset_limits():
    """The large-tile and decode kernels address their operands with 32-bit
    buffer offsets and are taken only below 2^31 bytes: A of 262143 x 16384
    (2^31 - 8 KiB of codes) through the large-tile kernel, and W of 262079
    rows x 16384 through the decode kernel, checked on the last rows and
    columns.  Tensor scales are given, so the oracle needs only the samples."""
    dev = need_gpu()
    K = 16384
    g = torch.tensor([0.0025], device=dev)
    gen = torch.Generator(device=dev).manual_seed(91)
    # large-tile kernel: M x K/2 = 2^31 - 8192, N = 256 (1024 tiles of 256 x 256)
    M, N = 262143, 256
    print(f"[gemm] large-tile kernel at its limit: A {M}x{K}, W {N}x{K}", flush=True)
    x = torch.randn((M, K), generator=gen, device=dev, dtype=torch.bfloat16)
    a = nv.quantize(x, g, from_amax=False)
    w = normal_weights(N, K, 0.02, seed=92, device=dev)
    b = nv.quantize(w)
    y = nv.gemm(*a, *b, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.array([0, 131072, M - 256, M - 2, M - 1])
    rows_t = torch.from_numpy(rows).to(dev)
    oa = ref.quantize(host_f32(x[rows_t]), g=np.float32(0.0025))
    ow = ref.quantize(host_f32(w))
    Y, S = ref.gemm_ref(*oa, *ow)
    assert_gemm_close(y[rows_t], Y, S, "large-tile kernel, last rows")
    del x, a, y
    # decode kernel: (N + 64) x K/2 = 2^31 - 8192, M = 3
    M, N = 3, 262079
    print(f"[gemm] decode kernel at its limit: A {M}x{K}, W {N}x{K}", flush=True)
    x = torch.randn((M, K), generator=gen, device=dev, dtype=torch.bfloat16)
    a = nv.quantize(x)
    w = torch.randn((N, K), generator=gen, device=dev, dtype=torch.bfloat16)
    b = nv.quantize(w, g, from_amax=False)
    y = nv.gemm(*a, *b, out_dtype=torch.float32)
    torch.cuda.synchronize()
    cols = np.array([0, 131040, N - 64, N - 2, N - 1])
    cols_t = torch.from_numpy(cols).to(dev)
    oa = ref.quantize(host_f32(x))
    assert float(a[2].item()) == float(oa[2])
    ow = ref.quantize(host_f32(w[cols_t]), g=np.float32(0.0025))
    assert np.array_equal(b[0][cols_t].cpu().numpy(), ow[0]) and np.array_equal(b[1][cols_t].cpu().numpy(), ow[1])
    Y, S = ref.gemm_ref(*oa, *ow)
    assert_gemm_close(y[:, cols_t], Y, S, "decode kernel, last weight rows")
