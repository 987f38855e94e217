"""GPU parity of the tail split of the large-tile GEMM: shapes whose 256 x 256
tile count leaves the last round of 256 workgroups at most a quarter full
split those tiles over K, keep fp32 partial sums in the workspace and add
them in a second kernel.  The tiles that take this path are found with the
tile walk written out below, and their outputs are checked on every element:
bit for bit through a selection weight (each output one exact product), and
against the fp64 oracle within the GEMM bound on ragged shapes, plain and
segmented, with K parts of unequal length."""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_05_amd as nv
from oracle import nvfp4_ref as ref
from tests.gpu_util import assert_gemm_close, gpu_f32, gpu_u8, need_gpu

pytestmark = pytest.mark.gpu


def _tile_coords(bid, tiles_m, tiles_n):
    """Tile of workgroup `bid` in the large-tile walk: ids dealt round-robin
    to 8 XCDs are regrouped per XCD into contiguous ranges, which are walked
    in groups of 8 tile rows."""
    ntiles = tiles_m * tiles_n
    per, rem = divmod(ntiles, 8)
    x, i = bid % 8, bid // 8
    t = x * (per + 1) + i if x < rem else rem * (per + 1) + (x - rem) * per + i
    group = 8 * tiles_n
    first_m = (t // group) * 8
    gsize = min(tiles_m - first_m, 8)
    r = t % group
    return first_m + r % gsize, r // gsize


def _tail_tiles(M, N):
    tm, tn = (M + 255) // 256, (N + 255) // 256
    tiles = tm * tn
    tail = tiles % 256
    assert tiles >= 256 and 0 < tail <= 64, "not a tail-split shape"
    out = [_tile_coords(b, tm, tn) for b in range(tiles - tail, tiles)]
    assert len(set(out)) == tail
    return out


def test_tile_walk_covers_every_tile_once():
    """The walk written out above is a bijection on the tiles (host check of
    the test's own helper)."""
    for tm, tn in ((16, 49), (17, 16), (9, 29), (1, 300)):
        seen = {_tile_coords(b, tm, tn) for b in range(tm * tn)}
        assert len(seen) == tm * tn and all(0 <= a < tm and 0 <= b < tn for a, b in seen)


def _random_nvfp4(rows, k, seed, scale_lo=0x28, scale_hi=0x48):
    """Random valid NVFP4 operand: every code, scales in [scale_lo, scale_hi)."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    scales = rng.integers(scale_lo, scale_hi, size=(rows, k // 16), dtype=np.uint8)
    return codes, scales


def _workspace_bytes(M, N, K):
    return nv.load().nvfp4_gemm_workspace_size(M, N, K, 0)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_split_tail_dequantizes_exactly(dt):
    """Selection weight (W row n = code 2 at column n % K, scale 1.0, g = 1):
    y[m, n] = deq(A)[m, n % K] bit for bit, also in the split tiles, where
    the product sits in one K part and every other part adds +0.  A runs
    through every (code, scale) pair.  4096 x 12384, K = 4608: 784 tiles, the
    last 16 split into 8 parts of 4 or 5 K steps."""
    need_gpu()
    M, N, K = 4096, 12384, 4608
    assert _workspace_bytes(M, N, K) == 16 * 8 * 256 * 256 * 4
    nb = K // 16
    codes = ((np.arange(K)[None, :] + np.arange(M)[:, None]) % 16).astype(np.uint8)
    scales = ((np.arange(M)[:, None] * nb + np.arange(nb)[None, :]) % 127).astype(np.uint8)
    ac = ref.pack_codes(codes)
    wcodes = np.zeros((N, K), np.uint8)
    wcodes[np.arange(N), np.arange(N) % K] = 2
    y = nv.gemm(gpu_u8(ac), gpu_u8(scales), gpu_f32(1.0), gpu_u8(ref.pack_codes(wcodes)),
                gpu_u8(np.full((N, nb), 0x38, np.uint8)), gpu_f32(1.0), out_dtype=dt)
    torch.cuda.synchronize()
    deq = ref.dequantize(ac, scales, 1.0)
    got = y.float().cpu().numpy()
    for tm, tn in _tail_tiles(M, N) + [(0, 0), (15, 48)]:
        r0, c0 = 256 * tm, 256 * tn
        rows, cols = np.arange(r0, min(r0 + 256, M)), np.arange(c0, min(c0 + 256, N))
        want = (deq[rows][:, cols % K] + 0.0).astype(np.float32)  # -0 -> +0
        blk = got[rows][:, cols]
        bad = np.argwhere(blk.view(np.uint32) != want.view(np.uint32))
        assert bad.size == 0, f"tile ({tm}, {tn}) {dt}: {len(bad)} outputs differ, first {bad[:3].tolist()}"


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("segmented", [False, True])
def test_split_tail_matches_oracle_on_ragged_shape(dt, segmented):
    """M = 4059, N = 12334 (ragged last tile row and column), K = 2944 (23 K
    steps in 5 parts of 4 or 5): every output of every split tile, and of two
    whole tiles, within the GEMM bound of the fp64 oracle.  Segmented: three
    modules, one boundary inside the last tile column."""
    need_gpu()
    M, N, K = 4059, 12334, 2944
    assert _workspace_bytes(M, N, K) == 16 * 5 * 256 * 256 * 4
    ac, as_ = _random_nvfp4(M, K, 11)
    wc, ws = _random_nvfp4(N, K, 12, 0x30, 0x40)
    g_a = np.float32(3.0517578e-05)
    module_rows = [6000, 6300, 34] if segmented else [N]
    gs = [np.float32(0.0021), np.float32(0.00037), np.float32(0.0123)][:len(module_rows)]
    gs_dev = torch.tensor([float(g) for g in gs], dtype=torch.float32, device="cuda")
    if segmented:
        y = nv.gemm_segmented(gpu_u8(ac), gpu_u8(as_), gpu_f32(g_a), gpu_u8(wc), gpu_u8(ws), gs_dev, module_rows,
                              out_dtype=dt)
    else:
        y = nv.gemm(gpu_u8(ac), gpu_u8(as_), gpu_f32(g_a), gpu_u8(wc), gpu_u8(ws), gs_dev[0:1], out_dtype=dt)
    torch.cuda.synchronize()
    ends = np.cumsum(module_rows)
    for tm, tn in _tail_tiles(M, N) + [(0, 0), (15, 48)]:
        rows = np.arange(256 * tm, min(256 * tm + 256, M))
        cols = np.arange(256 * tn, min(256 * tn + 256, N))
        # the oracle over these columns, module by module
        Y = np.zeros((len(rows), len(cols)))
        S = np.zeros_like(Y)
        for mi, (lo, hi) in enumerate(zip(np.concatenate([[0], ends[:-1]]), ends)):
            sel = (cols >= lo) & (cols < hi)
            if sel.any():
                Ym, Sm = ref.gemm_ref(ac[rows], as_[rows], g_a, wc[cols[sel]], ws[cols[sel]], gs[mi])
                Y[:, sel], S[:, sel] = Ym, Sm
        got = y[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()]
        assert_gemm_close(got, Y, S, f"tile ({tm}, {tn}) {'segmented' if segmented else 'plain'} {dt}")


def test_split_tail_is_deterministic_and_uses_the_given_workspace():
    """Two calls give the same bytes, also when the workspace holds garbage
    from an unrelated use (its contents need no initialisation)."""
    need_gpu()
    M, N, K = 4352, 4096, 1024   # 17 x 16 = 272 tiles: 16 split into 2 parts
    ac, as_ = _random_nvfp4(M, K, 21)
    wc, ws = _random_nvfp4(N, K, 22)
    args = (gpu_u8(ac), gpu_u8(as_), gpu_f32(0.01), gpu_u8(wc), gpu_u8(ws), gpu_f32(0.02))
    y1 = nv.gemm(*args, out_dtype=torch.bfloat16)
    junk = torch.full((_workspace_bytes(M, N, K) // 4,), float("nan"), device="cuda")
    del junk  # the allocator hands the same block to the next workspace
    y2 = nv.gemm(*args, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
