"""NVFP4 reference: plain numpy fp64, obviously correct, slow.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): imported by tests,
``smoke()`` and the CPU baseline of ``bench.py``, never by the product path.

What NVFP4 is, per [PX] (item 1 of "Background"): every value is a 4-bit E2M1
float; each run of 16 consecutive values carries one E4M3 scale chosen as the
block's absolute maximum divided by 6 (6 is the largest E2M1 magnitude); the
whole tensor carries one FP32 scale.  [LIT] ("Standing in the anthology")
contrasts it with MX: 16-element blocks with an E4M3 scale instead of
32-element blocks with a power-of-two scale.

Readings where the pages are silent (each one is a convention of this oracle):
  * The tensor scale g multiplies on dequantization: x ~ code * scale * g, and
    g = RN32(amax / (6 * 448)), i.e. the block scale of the block holding the
    tensor's absolute maximum lands on the E4M3 maximum 448.
  * The block scale is E4M3 round-to-nearest-even of the exact real number
    blockmax / (6 g), saturated at 448; E4M3 subnormals are kept and 0 is a
    legal scale.
  * Each code is E2M1 round-to-nearest-even of the exact real |x| / (scale g),
    saturated at 6, with the sign bit copied from x (so -0.0 and small
    negatives encode as 0x8; parity unpinned: a convention, dequantization is
    the same either way).  A zero scale gives all-zero magnitudes.
  * amax == 0 (or a quotient that underflows fp32 to 0) gives g = 1.0
    (parity unpinned: a convention).
  * Two codes per byte, the even column in the low nibble; codes are
    [rows, cols/2] and scales [rows, cols/16], both row-major; blocks run
    along the contraction dimension K of both GEMM operands.

Exactness.  Every rounding decision compares |x| (or the block max) against a
midpoint of the target grid times the divisor.  Those products have at most
31 significant bits (midpoint <= 5 bits, E4M3 scale <= 4 bits, 6 = 2 bits,
g = 24 bits), so they are exact in fp64, and so are the comparisons: the
rounding below is the exact-real definition, not an approximation of it.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# Grids.  E2M1: sign-magnitude, 2 exponent bits (bias 1), 1 mantissa bit.
# E4M3 ("fn" variant): 4 exponent bits (bias 7), 3 mantissa bits, no infinity,
# 0x7F is NaN, so the largest finite magnitude is 0x7E = 448.
# ----------------------------------------------------------------------------

def _e2m1_value(m: int) -> float:
    e, f = m >> 1, m & 1
    return f * 0.5 if e == 0 else (1.0 + f / 2.0) * 2.0 ** (e - 1)


def _e4m3_value(c: int) -> float:
    e, f = c >> 3, c & 7
    return f * 2.0 ** -9 if e == 0 else (1.0 + f / 8.0) * 2.0 ** (e - 7)


E2M1_VALUES = np.array([_e2m1_value(m) for m in range(8)], dtype=np.float64)
E2M1_MIDPOINTS = (E2M1_VALUES[:-1] + E2M1_VALUES[1:]) / 2.0
E4M3_MAX_CODE = 0x7E
E4M3_VALUES = np.array([_e4m3_value(c) for c in range(E4M3_MAX_CODE + 1)], dtype=np.float64)
E4M3_MIDPOINTS = (E4M3_VALUES[:-1] + E4M3_VALUES[1:]) / 2.0
E2M1_MAX = 6.0
E4M3_MAX = 448.0
GLOBAL_DIVISOR = E2M1_MAX * E4M3_MAX  # 2688
BLOCK = 16


def e4m3_decode(codes) -> np.ndarray:
    """Value of E4M3 scale bytes (0..0x7E) as fp64."""
    codes = np.asarray(codes, dtype=np.int64)
    if np.any((codes < 0) | (codes > E4M3_MAX_CODE)):
        raise ValueError("E4M3 scale byte out of range 0..0x7E")
    return E4M3_VALUES[codes]


def e2m1_decode(codes) -> np.ndarray:
    """Signed value of 4-bit E2M1 codes (bit 3 = sign) as fp64."""
    codes = np.asarray(codes, dtype=np.int64)
    mag = E2M1_VALUES[codes & 7]
    return np.where(codes & 8, -mag, mag)


def _round_to_grid_index(num: np.ndarray, thresholds: np.ndarray) -> np.ndarray:
    """Index of the grid point nearest to num / d, ties to the even index.

    ``thresholds[..., j]`` holds midpoint_j * d for the divisor d of each
    element (exact in fp64), so the quotient never has to be formed.  The
    index is the number of midpoints lying strictly below num; when num sits
    exactly on the next midpoint the two neighbours tie and the even one wins.
    Anything above the last midpoint takes the last grid point (saturation).
    """
    above = num[..., None] > thresholds
    idx = above.sum(axis=-1)
    n_mid = thresholds.shape[-1]
    nxt = np.take_along_axis(thresholds, np.minimum(idx, n_mid - 1)[..., None], axis=-1)[..., 0]
    tie = (idx < n_mid) & (num == nxt)
    return np.where(tie & (idx % 2 == 1), idx + 1, idx)


def global_scale(x) -> np.float32:
    """Per-tensor FP32 scale: RN32(amax / 2688); 1.0 when that is 0.

    [PX] gives one FP32 scale per tensor; the formula amax/(6*448) makes the
    block holding the tensor maximum use the top E4M3 scale.  numpy's float32
    division is IEEE correctly rounded, which is RN32 of the exact quotient.
    """
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("oracle input must be finite")
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    g = amax / np.float32(GLOBAL_DIVISOR)
    return np.float32(1.0) if g == 0 else np.float32(g)


def block_scales(x: np.ndarray, g: np.float32) -> np.ndarray:
    """E4M3 scale byte of every 16-element block: RNE(blockmax / (6 g)), saturated.

    [PX]: the block scale is set to blockmax/6 (in units of the tensor scale).
    Returns uint8 [rows, cols/16].
    """
    rows, cols = x.shape
    bm = np.abs(x.astype(np.float64)).reshape(rows, cols // BLOCK, BLOCK).max(axis=-1)
    thresholds = E4M3_MIDPOINTS * (6.0 * np.float64(g))  # exact: <= 31 significant bits
    idx = np.searchsorted(thresholds, bm, side="left")   # midpoints strictly below bm
    nxt = thresholds[np.minimum(idx, thresholds.size - 1)]
    tie = (idx < thresholds.size) & (bm == nxt)
    idx = np.where(tie & (idx % 2 == 1), idx + 1, idx)
    return idx.astype(np.uint8)


def element_codes(x: np.ndarray, scales: np.ndarray, g: np.float32) -> np.ndarray:
    """4-bit code of every element: sign | E2M1_RNE(|x| / (val(scale) g)), saturated.

    Returns uint8 [rows, cols] holding one code (0..15) per element.
    """
    rows, cols = x.shape
    xa = np.abs(x.astype(np.float64)).reshape(rows, cols // BLOCK, BLOCK)
    unit = e4m3_decode(scales) * np.float64(g)                     # exact: 28 bits
    thresholds = unit[..., None, None] * E2M1_MIDPOINTS             # exact: <= 31 bits
    thresholds = np.broadcast_to(thresholds, xa.shape + (E2M1_MIDPOINTS.size,))
    mag = _round_to_grid_index(xa, thresholds)
    mag = np.where(unit[..., None] == 0.0, 0, mag)                  # zero scale: all zero
    sign = np.signbit(x.reshape(rows, cols // BLOCK, BLOCK)).astype(np.int64)
    return ((sign << 3) | mag).reshape(rows, cols).astype(np.uint8)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Two codes per byte, even column in the low nibble: [rows, cols] -> [rows, cols/2]."""
    codes = codes.astype(np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    rows, half = packed.shape
    out = np.empty((rows, half * 2), dtype=np.uint8)
    out[:, 0::2] = packed & 0x0F
    out[:, 1::2] = packed >> 4
    return out


def quantize(x, g=None, chunk_rows: int = 4096):
    """NVFP4-quantize a [rows, cols] tensor (cols % 16 == 0).

    g=None computes the tensor scale from x (``global_scale``); otherwise g is
    the caller's positive finite fp32 tensor scale (calibrated, static).
    Returns (packed codes uint8 [rows, cols/2], scales uint8 [rows, cols/16], g).
    """
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] % BLOCK:
        raise ValueError("expected a [rows, cols] tensor with cols % 16 == 0")
    if not np.all(np.isfinite(x)):
        raise ValueError("oracle input must be finite")
    g = global_scale(x) if g is None else np.float32(g)
    if not (np.isfinite(g) and g > 0):
        raise ValueError("tensor scale must be positive and finite")
    rows, cols = x.shape
    codes = np.empty((rows, cols // 2), dtype=np.uint8)
    scales = np.empty((rows, cols // BLOCK), dtype=np.uint8)
    for r0 in range(0, rows, chunk_rows):
        xs = x[r0:r0 + chunk_rows]
        s = block_scales(xs, g)
        scales[r0:r0 + chunk_rows] = s
        codes[r0:r0 + chunk_rows] = pack_codes(element_codes(xs, s, g))
    return codes, scales, g


def dequantize(codes, scales, g, include_global: bool = True) -> np.ndarray:
    """fp64 values code * val(scale) (* g): exact, since every factor fits fp64."""
    c = e2m1_decode(unpack_codes(codes))
    rows, cols = c.shape
    s = e4m3_decode(scales)
    v = (c.reshape(rows, cols // BLOCK, BLOCK) * s[..., None]).reshape(rows, cols)
    return v * np.float64(g) if include_global else v


def gemm_ref(a_codes, a_scales, g_a, w_codes, w_scales, g_w):
    """Y = deq(A) deq(W)^T with A [M, K] and W [N, K], in fp64.

    Returns (Y, Sabs) where Sabs[m, n] = sum_k |deqA[m, k] deqW[n, k]|, the base
    of the per-element tolerance |y - Y| <= 1e-4 * Sabs.  Both operands carry
    their tensor scales, so Y is the W4A4 linear layer's output.
    """
    a = dequantize(a_codes, a_scales, g_a, include_global=False)
    w = dequantize(w_codes, w_scales, g_w, include_global=False)
    alpha = np.float64(g_a) * np.float64(g_w)   # exact: product of two fp32
    y = (a @ w.T) * alpha
    sabs = (np.abs(a) @ np.abs(w).T) * alpha
    return y, sabs


def gemm_segmented_ref(a_codes, a_scales, g_a, w_codes, w_scales, module_gs, module_rows):
    """One GEMM over modules concatenated along N in which every module keeps
    its own tensor scale: the columns of module i are g_a g_i deq(A) deq(W_i)^T.
    This is the per-module result that a fused projection must reproduce
    ([CT] "Main findings", last bullet; [LIT] "Standing in the anthology"),
    written as what it means: the per-module GEMMs side by side.

    Returns (Y, Sabs) like gemm_ref."""
    ys, ss = [], []
    r0 = 0
    for g_i, rows in zip(module_gs, module_rows):
        sl = slice(r0, r0 + int(rows))
        y, sabs = gemm_ref(a_codes, a_scales, g_a, w_codes[sl], w_scales[sl], np.float32(g_i))
        ys.append(y)
        ss.append(sabs)
        r0 += int(rows)
    if r0 != w_codes.shape[0]:
        raise ValueError("module rows must add up to the weight rows")
    return np.concatenate(ys, axis=1), np.concatenate(ss, axis=1)


def softplus(z) -> np.ndarray:
    """log(1 + e^z) in fp64, as max(z, 0) + log1p(e^-|z|) so that no
    exponential overflows."""
    z = np.asarray(z, dtype=np.float64)
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def sigmoid(z) -> np.ndarray:
    """1 / (1 + e^-z) in fp64, with the exponential taken of -|z| (no overflow)."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def silu(z) -> np.ndarray:
    """z * sigmoid(z) in fp64."""
    z = np.asarray(z, dtype=np.float64)
    return z * sigmoid(z)


def gemm_swiglu_ref(a_codes, a_scales, g_a, w_codes, w_scales, g_w):
    """The MLP gate/up projection followed by SwiGLU, fp64: with W = [gate (F
    rows); up (F rows)], Y = gemm_ref(A, W) and h = silu(Y_gate) * Y_up.  The
    activation between the two MLP projections is not on the pages; SwiGLU
    is the reading adopted for it.  Returns (H, G, U, SG, SU): h, the gate
    and up outputs, and their error allowances' Sabs from gemm_ref."""
    y, sabs = gemm_ref(a_codes, a_scales, g_a, w_codes, w_scales, g_w)
    f = y.shape[1] // 2
    g, u = y[:, :f], y[:, f:]
    return silu(g) * u, g, u, sabs[:, :f], sabs[:, f:]


def gdn_decay_gate(v, a_log, dt_bias) -> np.ndarray:
    """Log-space decay gate of a GDN head: g = -exp(A_log) * softplus(a + dt_bias)
    ([PX] "Gated DeltaNet Mechanics"); v holds the a-projection outputs
    [rows, heads], a_log and dt_bias one value per head.  The forget gate is
    alpha = exp(g), in (0, 1]."""
    v = np.asarray(v, dtype=np.float64)
    return -np.exp(np.asarray(a_log, dtype=np.float64)) * softplus(v + np.asarray(dt_bias, dtype=np.float64))


def gdn_write_gate(v) -> np.ndarray:
    """Write strength beta = sigmoid(b) of the b-projection outputs ([LIT]
    "Key takeaways", gates bullet: the sigmoid write strength)."""
    return sigmoid(v)


def gemm_segmented_gates_ref(a_codes, a_scales, g_a, w_codes, w_scales, module_gs, module_rows,
                             decay_module, a_log, dt_bias, write_module):
    """gemm_segmented_ref, then the GDN gates in the epilogue: the columns of
    module `decay_module` become gdn_decay_gate of their values (column j
    with a_log[j], dt_bias[j]), those of `write_module` gdn_write_gate; -1
    selects none.  Returns (G, Y, Sabs): the gated output, and the pre-gate
    output with its error allowance from gemm_ref."""
    y, sabs = gemm_segmented_ref(a_codes, a_scales, g_a, w_codes, w_scales, module_gs, module_rows)
    out = y.copy()
    starts = np.concatenate([[0], np.cumsum([int(r) for r in module_rows])])
    if decay_module >= 0:
        sl = slice(starts[decay_module], starts[decay_module + 1])
        out[:, sl] = gdn_decay_gate(y[:, sl], a_log, dt_bias)
    if write_module >= 0:
        sl = slice(starts[write_module], starts[write_module + 1])
        out[:, sl] = gdn_write_gate(y[:, sl])
    return out, y, sabs


def harmonize_ref(scales_list, module_gs):
    """Bring per-module tensor scales of a fused projection to one shared scale.

    [CT] (last bullet of "Main findings") and [LIT] ("Standing in the
    anthology"): when modules calibrated each with their own FP32 tensor scale
    are served as one fused GEMM, one tensor scale is applied to all of them
    and the small gate projections come out mis-scaled; the released weights
    are re-expressed under one shared scale.  The pages do not give the
    procedure; the reading used here: shared g* = max_i g_i (so no rescaled
    block scale can exceed the E4M3 range) and every block scale of module i
    becomes E4M3_RNE(val(s) g_i / g*), exact real quotient, saturated; codes
    are unchanged.

    Returns (harmonized scales [sum rows, K/16] uint8, g*, n_inexact,
    n_subnormal) where n_inexact counts blocks with val(s') g* != val(s) g_i
    and n_subnormal counts nonzero input scales whose result has a zero
    exponent field (E4M3 subnormal, or flushed to zero).
    """
    gs = [np.float32(g) for g in module_gs]
    if any(not (np.isfinite(g) and g > 0) for g in gs):
        raise ValueError("module scales must be positive and finite")
    g_star = max(gs)
    thresholds = E4M3_MIDPOINTS * np.float64(g_star)        # exact: <= 29 bits
    out, n_inexact, n_sub = [], 0, 0
    for s, g in zip(scales_list, gs):
        s = np.asarray(s, dtype=np.uint8)
        target = e4m3_decode(s) * np.float64(g)              # exact: <= 28 bits
        idx = np.searchsorted(thresholds, target, side="left")
        nxt = thresholds[np.minimum(idx, thresholds.size - 1)]
        tie = (idx < thresholds.size) & (target == nxt)
        idx = np.where(tie & (idx % 2 == 1), idx + 1, idx).astype(np.uint8)
        n_inexact += int(np.count_nonzero(E4M3_VALUES[idx] * np.float64(g_star) != target))
        n_sub += int(np.count_nonzero((s != 0) & ((idx >> 3) == 0)))
        out.append(idx)
    return np.concatenate(out, axis=0), np.float32(g_star), n_inexact, n_sub


def naive_fused_ref(a_codes, a_scales, g_a, w_codes, w_scales, module_gs):
    """The broken serving case: one fused GEMM over concatenated module weights
    that applies the first module's tensor scale to every column ([LIT],
    "Standing in the anthology": the gates computed with mis-scaled weights).
    Which single scale a fused kernel uses is not on the pages; the first
    module's (qkv in a GDN in-projection) is this oracle's convention
    (parity unpinned)."""
    return gemm_ref(a_codes, a_scales, g_a, w_codes, w_scales, np.float32(module_gs[0]))
