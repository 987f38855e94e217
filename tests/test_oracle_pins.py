"""Pins of the CPU oracle to things other than itself (CPU only).

Each test checks the fp64 oracle against something the NVFP4 definition or
mathematics fixes: hand-worked blocks, closed forms, torch's float8 cast,
invariants that hold for any input, brute force over every (code, scale), and
the independent exact-rational twin.
"""
import json
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import exact
from oracle import nvfp4_ref as ref


def _f32(v):
    return struct.unpack("<f", struct.pack("<f", v))[0]


# ------------------------------------------------------------------ golden
def _golden(golden_dir):
    with open(os.path.join(golden_dir, "hand_blocks.json")) as f:
        return json.load(f)["blocks"]


def test_hand_worked_blocks(golden_dir):
    for blk in _golden(golden_dir):
        x = np.array([blk["x"]], dtype=np.float32)
        codes, scales, g = ref.quantize(x, g=blk["g"])
        if "g_expected_hex" in blk:
            want = int(blk["g_expected_hex"][:8], 16)
            assert int(np.float32(g).view(np.uint32)) == want, blk["name"]
            continue
        if "g_expected" in blk:
            assert g == np.float32(blk["g_expected"]), blk["name"]
        assert scales[0, 0] == int(blk["scale"], 16), blk["name"]
        assert bytes(codes[0]).hex().upper() == blk["packed"], blk["name"]
        # the exact twin agrees on every hand-worked block
        s_ex, c_ex = exact.quantize_block_exact([float(v) for v in x[0]], float(g))
        assert s_ex == scales[0, 0], blk["name"]
        assert c_ex == list(ref.unpack_codes(codes)[0]), blk["name"]


def test_h1_round_trip_is_exact(golden_dir):
    blk = _golden(golden_dir)[0]
    x = np.array([blk["x"]], dtype=np.float32)
    c, s, g = ref.quantize(x, g=1.0)
    d = ref.dequantize(c, s, g)
    assert np.array_equal(d, x.astype(np.float64))
    assert np.array_equal(np.signbit(d), np.signbit(x))


def test_negative_zero_and_small_negatives_keep_sign():
    x = np.zeros((1, 16), dtype=np.float32)
    x[0, 0] = 6.0
    x[0, 1] = -0.0
    x[0, 2] = -0.1
    c, s, g = ref.quantize(x, g=1.0)
    codes = ref.unpack_codes(c)[0]
    assert codes[1] == 8 and codes[2] == 8 and codes[3] == 0


# ------------------------------------------------------------ closed forms
def test_e2m1_grid_closed_form():
    assert list(ref.E2M1_VALUES) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(ref.E2M1_MIDPOINTS) == [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    assert ref.GLOBAL_DIVISOR == 2688.0
    for c in range(16):
        v = ref.e2m1_decode([c])[0]
        assert (v < 0) == bool(c & 8) or v == 0
        assert abs(v) == ref.E2M1_VALUES[c & 7]


def test_e4m3_decode_matches_torch_float8():
    codes = torch.arange(0, 0x7F, dtype=torch.uint8)
    want = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = ref.e4m3_decode(np.arange(0, 0x7F))
    assert np.array_equal(got, want)
    assert ref.e4m3_decode([0x38])[0] == 1.0
    assert ref.e4m3_decode([0x7E])[0] == 448.0
    assert ref.e4m3_decode([0x01])[0] == 2.0 ** -9
    with pytest.raises(ValueError):
        ref.e4m3_decode([0x7F])


def test_e4m3_rounding_matches_torch_cast():
    """Block-scale rounding = torch's fp32->float8_e4m3fn cast after clamping at
    448 (torch returns NaN past 464).  With g = 1/2 the divisor 6g = 3, and
    blockmax = 3q is exact for q with <= 22 significant bits, so the oracle
    rounds the exact real q."""
    rng = np.random.default_rng(11)
    q = np.concatenate([
        np.exp2(rng.uniform(-13, 9.2, 20000)),
        ref.E4M3_MIDPOINTS,                       # every tie
        np.nextafter(ref.E4M3_MIDPOINTS, 0), np.nextafter(ref.E4M3_MIDPOINTS, 1e9),
        [448.0, 460.0, 464.0, 470.0, 480.0, 1000.0, 2.0 ** -10, 1.5 * 2.0 ** -10],
    ]).astype(np.float32)
    q = q.view(np.uint32) & np.uint32(0xFFFFFFFC)           # <= 22 significant bits
    q = q.view(np.float32)
    bm = (q.astype(np.float64) * 3.0).astype(np.float32)
    assert np.array_equal(bm.astype(np.float64), q.astype(np.float64) * 3.0)
    x = np.zeros((q.size, 16), dtype=np.float32)
    x[:, 0] = bm
    _, s, _ = ref.quantize(x, g=0.5)
    want = torch.from_numpy(np.minimum(q, 448.0)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(s[:, 0], want)


def test_global_scale_is_rn32_of_exact_quotient():
    rng = np.random.default_rng(5)
    for _ in range(300):
        x = (rng.standard_normal(64) * 10.0 ** rng.uniform(-6, 6)).astype(np.float32)
        g = ref.global_scale(x)
        assert g == np.float32(exact.global_scale_exact([float(v) for v in x]))
    assert ref.global_scale(np.zeros(32, np.float32)) == np.float32(1.0)
    assert ref.global_scale(np.array([2688.0, -5.0], np.float32)) == np.float32(1.0)


# ---------------------------------------------------------------- invariants
def _heavy(rows, cols, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, size=(rows, cols)).astype(np.float32)
    ch = rng.choice(cols, max(1, cols // 100), replace=False)
    x[:, ch] *= 60
    return x


def test_invariant_block_max_maps_to_six():
    """I1: for a normal, unsaturated block scale the block maximum gets code +-6:
    blockmax/(s g) lies in [6/(1+2^-4), 6/(1-2^-4)], above the midpoint 5."""
    x = _heavy(64, 512, 1)
    c, s, g = ref.quantize(x)
    codes = ref.unpack_codes(c).reshape(64, 32, 16)
    xa = np.abs(x).reshape(64, 32, 16)
    arg = xa.argmax(axis=-1)
    top = np.take_along_axis(codes, arg[..., None], axis=-1)[..., 0]
    normal = (s >> 3) > 0
    unsat = s < 0x7E
    sel = normal & unsat
    assert sel.sum() > 1000
    assert np.all((top[sel] & 7) == 7)


def test_invariant_error_bound():
    """I2: |x - deq| <= half an E2M1 step times val(s) g (saturated blocks excluded)."""
    x = _heavy(64, 512, 2)
    c, s, g = ref.quantize(x)
    d = ref.dequantize(c, s, g)
    unit = (ref.e4m3_decode(s) * np.float64(g))[..., None]
    mag = np.abs(ref.e2m1_decode(ref.unpack_codes(c))).reshape(64, 32, 16)
    half = np.where(mag < 2, 0.25, np.where(mag < 4, 0.5, 1.0))
    err = np.abs(x.astype(np.float64) - d).reshape(64, 32, 16)
    ok = err <= half * unit
    ok |= (s == 0x7E)[..., None]
    assert np.all(ok)


def test_invariant_scale_equivariance():
    """I3: multiplying x and g by 2^k changes neither codes nor scales."""
    x = _heavy(16, 256, 3)
    c0, s0, g0 = ref.quantize(x)
    for k in (-20, -3, 1, 7):
        c1, s1, g1 = ref.quantize(x * np.float32(2.0 ** k), g=np.float32(g0 * 2.0 ** k))
        assert np.array_equal(c0, c1) and np.array_equal(s0, s1)
        assert g1 == ref.global_scale(x * np.float32(2.0 ** k))


def test_invariant_products_exact_in_bf16_and_fp16():
    """I4: every E2M1 value times every E4M3 scale is exact in bf16 and fp16."""
    prod = ref.E2M1_VALUES[:, None] * ref.E4M3_VALUES[None, :]
    t = torch.from_numpy(prod)
    assert torch.equal(t.to(torch.bfloat16).double(), t)
    assert torch.equal(t.to(torch.float16).double(), t)


def test_invariant_amax_order_independent():
    """I5: the tensor scale does not depend on element order."""
    x = _heavy(8, 256, 4)
    rng = np.random.default_rng(0)
    g0 = ref.global_scale(x)
    for _ in range(5):
        assert ref.global_scale(rng.permutation(x.ravel()).reshape(x.shape)) == g0


# ---------------------------------------------------------------- brute force
def test_brute_force_every_scale_and_code_round_trips():
    """P5: a block [6 val(s), V[m] val(s), 0...] returns scale s and codes 7, m."""
    rows = []
    expect = []
    for s in range(1, 0x7F):
        vs = ref.E4M3_VALUES[s]
        for m in range(16):
            row = np.zeros(16, np.float64)
            row[0] = 6.0 * vs
            row[1] = ref.e2m1_decode([m])[0] * vs
            if m == 8:
                row[1] = -0.0
            rows.append(row)
            expect.append((s, m))
    x = np.array(rows, dtype=np.float32)
    assert np.array_equal(x.astype(np.float64), np.array(rows))
    c, sc, _ = ref.quantize(x, g=1.0)
    codes = ref.unpack_codes(c)
    for i, (s, m) in enumerate(expect):
        assert sc[i, 0] == s and codes[i, 0] == 7 and codes[i, 1] == m, (s, m)


def test_brute_force_every_bf16_pattern_beside_fixed_max():
    """Every finite bf16 bit pattern as one element of a block whose max is 96
    (scale 16 = 0x58), checked element by element against the exact twin."""
    pats = np.arange(0, 1 << 16, dtype=np.uint32)
    vals = (pats << 16).view(np.float32)
    keep = np.isfinite(vals) & (np.abs(vals) <= 96.0)
    vals = vals[keep]
    x = np.zeros((vals.size, 16), np.float32)
    x[:, 0] = 96.0
    x[:, 1] = vals
    c, s, _ = ref.quantize(x, g=1.0)
    assert np.all(s[:, 0] == 0x58)
    codes = ref.unpack_codes(c)[:, 1]
    unit = Fraction(16)
    for v, got in zip(vals.tolist(), codes.tolist()):
        sign = 8 if np.signbit(np.float32(v)) else 0
        want = sign | exact.nearest_even(abs(Fraction(v)) / unit, exact.E2M1)
        assert got == want, v


def test_fp64_oracle_matches_exact_twin_random_and_near_ties():
    rng = np.random.default_rng(7)
    blocks = []
    # random heavy-tailed blocks with random tensor scales
    for _ in range(3000):
        blocks.append((rng.standard_t(3, 16) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32))
    # engineered near-ties: elements at and 1 ulp around every E2M1 midpoint of a block
    for s in (0x30, 0x38, 0x3B, 0x47, 0x55, 0x05):
        for gi in (np.float32(1.0), np.float32(0.3), np.float32(1.7e-3)):
            unit = ref.E4M3_VALUES[s] * np.float64(gi)
            for mid in ref.E2M1_MIDPOINTS:
                t = np.float32(mid * unit)
                row = np.array([np.float32(6 * unit), t, np.nextafter(t, np.float32(0)),
                                np.nextafter(t, np.float32(1e30)), -t,
                                -np.nextafter(t, np.float32(0)), 0, 0, 0, 0, 0, 0, 0, 0, 0, 0],
                               dtype=np.float32)
                blocks.append((row, gi))
    for item in blocks:
        if isinstance(item, tuple):
            row, gi = item
        else:
            row, gi = item, ref.global_scale(item) * np.float32(rng.uniform(0.5, 2.0))
        c, s, g = ref.quantize(row[None, :], g=gi)
        s_ex, c_ex = exact.quantize_block_exact([float(v) for v in row], float(g))
        assert s[0, 0] == s_ex
        assert list(ref.unpack_codes(c)[0]) == c_ex


def test_fp64_oracle_matches_exact_twin_at_scale_ties():
    """Block maxima at and 1 ulp around every E4M3 midpoint times 6g."""
    for gi in (np.float32(1.0), np.float32(0.37), np.float32(3.1e-4)):
        for mid in ref.E4M3_MIDPOINTS:
            t = np.float32(mid * 6.0 * np.float64(gi))
            for v in (t, np.nextafter(t, np.float32(0)), np.nextafter(t, np.float32(1e30))):
                row = np.zeros((1, 16), np.float32)
                row[0, 3] = v
                row[0, 4] = -v / 3
                c, s, g = ref.quantize(row, g=gi)
                s_ex, c_ex = exact.quantize_block_exact([float(u) for u in row[0]], float(gi))
                assert s[0, 0] == s_ex
                assert list(ref.unpack_codes(c)[0]) == c_ex


# ------------------------------------------------------------------- GEMM
def _quant(x, g=None):
    return ref.quantize(np.asarray(x, np.float32), g=g)


def test_gemm_against_exact_sums_tiny_config_slice():
    """P6: the fp64 GEMM equals exact rational sums to within K 2^-53 Sabs."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    x[:, [5, 77]] *= 50
    w = (rng.standard_normal((24, 256)) * 0.02).astype(np.float32)
    ac, as_, ga = _quant(x)
    wc, ws, gw = _quant(w)
    y, sabs = ref.gemm_ref(ac, as_, ga, wc, ws, gw)
    ex = exact.gemm_exact(ref.unpack_codes(ac).tolist(), as_.tolist(), float(ga),
                          ref.unpack_codes(wc).tolist(), ws.tolist(), float(gw))
    for m in range(4):
        for n in range(24):
            assert abs(Fraction(float(y[m, n])) - ex[m][n]) <= Fraction(256 * 2.0 ** -52) * Fraction(float(sabs[m, n])) + Fraction(1, 10 ** 300)


def test_gemm_orientation_and_scales_against_loops():
    """Non-square shapes: Y[m, n] = sum_k A[m, k] W[n, k] g_a g_w, by explicit loops
    (catches a transposed operand, a dropped tensor scale or a sign error)."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 48)).astype(np.float32)
    w = rng.standard_normal((5, 48)).astype(np.float32) * 0.1
    ac, as_, ga = _quant(x)
    wc, ws, gw = _quant(w, g=np.float32(0.0123))
    y, sabs = ref.gemm_ref(ac, as_, ga, wc, ws, gw)
    A = ref.unpack_codes(ac)
    W = ref.unpack_codes(wc)
    for m in range(3):
        for n in range(5):
            acc = 0.0
            sab = 0.0
            for k in range(48):
                a = float(exact.dequant_exact(int(A[m, k]), int(as_[m, k // 16]), float(ga)))
                b = float(exact.dequant_exact(int(W[n, k]), int(ws[n, k // 16]), float(gw)))
                acc += a * b
                sab += abs(a * b)
            assert abs(y[m, n] - acc) <= 1e-12 * sab
            assert abs(sabs[m, n] - sab) <= 1e-12 * sab
    assert y.shape == (3, 5)


def test_gemm_identity_weight_reproduces_dequantized_activations():
    """P7: W = I (code 2 = 1.0, scale 0x38, g_w = 1) gives Y = deq(A) exactly."""
    rng = np.random.default_rng(2)
    x = rng.standard_t(3, (8, 64)).astype(np.float32)
    ac, as_, ga = _quant(x)
    eye_codes = (np.eye(64, dtype=np.uint8) * 2)          # code 2 = 1.0 on the diagonal
    wc = ref.pack_codes(eye_codes)
    ws = np.full((64, 4), 0x38, np.uint8)                  # every block scale 1.0
    assert np.array_equal(ref.dequantize(wc, ws, 1.0), np.eye(64))
    y, _ = ref.gemm_ref(ac, as_, ga, wc, ws, np.float32(1.0))
    assert np.array_equal(y, ref.dequantize(ac, as_, ga))


# --------------------------------------------------------------- harmonize
def _modules(seed, mults=(1.0, 1.0, 1.0, 1.0)):
    rng = np.random.default_rng(seed)
    sizes = (32, 16, 4, 4)
    out = []
    for r, mlt in zip(sizes, mults):
        w = (rng.standard_normal((r, 128)) * 0.02 * mlt).astype(np.float32)
        out.append(_quant(w))
    return out


def test_harmonize_power_of_two_ratios_are_exact():
    mods = _modules(3)
    base = mods[0][2]
    gs = [base, np.float32(base / 2), np.float32(base / 8), np.float32(base * 2)]
    scales = [m[1] for m in mods]
    # rescaling by a power of two ratio (no subnormal results) is exact
    new, g_star, n_inexact, n_sub = ref.harmonize_ref(scales, gs)
    assert g_star == np.float32(base * 2)
    assert n_inexact == 0 and n_sub == 0
    row = 0
    for s, g in zip(scales, gs):
        v_old = ref.e4m3_decode(s) * np.float64(g)
        v_new = ref.e4m3_decode(new[row:row + s.shape[0]]) * np.float64(g_star)
        assert np.array_equal(v_old, v_new)
        row += s.shape[0]


def test_harmonize_general_ratios_bounded_and_matches_exact_twin():
    mods = _modules(4, mults=(1.0, 1.3, 4.0, 0.25))
    scales = [m[1] for m in mods]
    gs = [m[2] for m in mods]
    new, g_star, n_inexact, n_sub = ref.harmonize_ref(scales, gs)
    assert g_star == max(gs)
    row = 0
    cnt = 0
    for s, g in zip(scales, gs):
        for r in range(s.shape[0]):
            for j in range(s.shape[1]):
                want = exact.harmonize_scale_exact(int(s[r, j]), float(g), float(g_star))
                assert new[row + r, j] == want
                v_old = Fraction(float(ref.E4M3_VALUES[s[r, j]])) * Fraction(float(g))
                v_new = Fraction(float(ref.E4M3_VALUES[want])) * Fraction(float(g_star))
                if v_new != v_old:
                    cnt += 1
                if want >= 8:   # normal result: within half an E4M3 step (2^-4 relative)
                    assert abs(v_new - v_old) <= v_old / 16
        row += s.shape[0]
    assert cnt == n_inexact and n_inexact > 0


def test_naive_fused_closed_form():
    """Naive fused GEMM: column block i equals the per-module result times g_1/g_i."""
    rng = np.random.default_rng(9)
    x = rng.standard_t(3, (4, 128)).astype(np.float32)
    ac, as_, ga = _quant(x)
    mods = _modules(5, mults=(1.0, 2.0, 5.0, 0.3))
    wc = np.concatenate([m[0] for m in mods])
    ws = np.concatenate([m[1] for m in mods])
    gs = [m[2] for m in mods]
    y_naive, _ = ref.naive_fused_ref(ac, as_, ga, wc, ws, gs)
    row = 0
    for (c, s, g) in mods:
        y_i, _ = ref.gemm_ref(ac, as_, ga, c, s, g)
        blk = y_naive[:, row:row + c.shape[0]]
        assert np.allclose(blk, y_i * (np.float64(gs[0]) / np.float64(g)), rtol=1e-12, atol=0)
        row += c.shape[0]


# ------------------------------------------------------- segmented epilogue
def test_segmented_gemm_column_loop_with_ragged_and_empty_modules():
    """Each output column carries the tensor scale of the module its weight row
    came from, found here by repeating module indices (not by slicing): a wrong
    range boundary, an empty module or a dropped g_i fails."""
    rng = np.random.default_rng(11)
    x = rng.standard_t(3, (3, 64)).astype(np.float32)
    ac, as_, ga = _quant(x)
    rows = [3, 0, 5, 1]
    mults = [1.0, 7.0, 0.1, 40.0]
    parts = [_quant((rng.standard_normal((r, 64)) * 0.02 * m).astype(np.float32)) for r, m in zip(rows, mults)]
    wc = np.concatenate([p[0] for p in parts])
    ws = np.concatenate([p[1] for p in parts])
    gs = [p[2] for p in parts]
    y, sabs = ref.gemm_segmented_ref(ac, as_, ga, wc, ws, gs, rows)
    owner = np.repeat(np.arange(len(rows)), rows)
    A = ref.dequantize(ac, as_, 1.0, include_global=False)
    W = ref.dequantize(wc, ws, 1.0, include_global=False)
    assert y.shape == (3, sum(rows))
    for n in range(sum(rows)):
        g = np.float64(ga) * np.float64(gs[owner[n]])
        for m in range(3):
            terms = A[m] * W[n] * g
            assert abs(y[m, n] - terms.sum()) <= 1e-12 * np.abs(terms).sum()
            assert abs(sabs[m, n] - np.abs(terms).sum()) <= 1e-12 * np.abs(terms).sum()


def test_segmented_gemm_special_cases():
    """One module is the plain GEMM; modules sharing one scale are the plain
    GEMM of their concatenation; power-of-two ratios make the harmonized GEMM
    equal to the segmented one."""
    rng = np.random.default_rng(12)
    x = rng.standard_t(3, (4, 128)).astype(np.float32)
    ac, as_, ga = _quant(x)
    mods = _modules(6)
    wc = np.concatenate([m[0] for m in mods])
    ws = np.concatenate([m[1] for m in mods])
    rows = [m[0].shape[0] for m in mods]
    g = mods[0][2]
    y1, s1 = ref.gemm_segmented_ref(ac, as_, ga, wc, ws, [g], [sum(rows)])
    y0, s0 = ref.gemm_ref(ac, as_, ga, wc, ws, g)
    assert np.array_equal(y1, y0) and np.array_equal(s1, s0)
    y2, _ = ref.gemm_segmented_ref(ac, as_, ga, wc, ws, [g] * 4, rows)
    assert np.allclose(y2, y0, rtol=1e-13, atol=1e-300)
    gs = [g, np.float32(g / 2), np.float32(g / 8), np.float32(g * 2)]
    # re-quantize each module with its own power-of-two-related scale
    parts = [_quant((rng.standard_normal((r, 128)) * 0.02).astype(np.float32), g=gi) for r, gi in zip(rows, gs)]
    wc = np.concatenate([p[0] for p in parts])
    hs, g_star, n_inexact, n_sub = ref.harmonize_ref([p[1] for p in parts], gs)
    assert n_inexact == 0 and n_sub == 0
    y_seg, s_seg = ref.gemm_segmented_ref(ac, as_, ga, wc, np.concatenate([p[1] for p in parts]), gs, rows)
    y_har, _ = ref.gemm_ref(ac, as_, ga, wc, hs, g_star)
    assert np.all(np.abs(y_seg - y_har) <= 1e-13 * s_seg)


# ------------------------------------------------------------------ GDN gates
def test_softplus_and_sigmoid_closed_forms_and_identities():
    import math
    assert abs(ref.softplus(0.0) - math.log(2.0)) < 1e-15
    z = np.linspace(-30.0, 30.0, 241)
    # softplus(z) - softplus(-z) = z; sigmoid(z) + sigmoid(-z) = 1
    assert np.allclose(ref.softplus(z) - ref.softplus(-z), z, rtol=0, atol=1e-12)
    assert np.allclose(ref.sigmoid(z) + ref.sigmoid(-z), 1.0, rtol=0, atol=1e-15)
    # sigmoid is the derivative of softplus (central differences)
    h = 1e-5
    assert np.allclose((ref.softplus(z + h) - ref.softplus(z - h)) / (2 * h), ref.sigmoid(z), rtol=0, atol=1e-9)
    assert ref.sigmoid(0.0) == 0.5
    assert abs(ref.sigmoid(math.log(3.0)) - 0.75) < 1e-15 and abs(ref.sigmoid(-math.log(3.0)) - 0.25) < 1e-15
    # asymptotes, without overflow
    with np.errstate(over="raise"):
        assert abs(ref.softplus(50.0) - 50.0) < 1e-14
        assert abs(ref.softplus(-50.0) / math.exp(-50.0) - 1.0) < 1e-12
        assert ref.sigmoid(1000.0) == 1.0 and ref.sigmoid(-1000.0) == 0.0


def test_decay_gate_closed_forms():
    import math
    dt = np.array([-6.9, -2.25, 0.0, 0.7, 3.0])
    # at a + dt_bias = 0 the gate is -exp(A_log) ln 2, whatever dt_bias is
    assert np.allclose(ref.gdn_decay_gate(-dt, np.zeros(5), dt), -math.log(2.0), rtol=0, atol=1e-15)
    # exp(A_log) multiplies: A_log = ln 2 doubles the gate
    v = np.array([[-3.0, -0.5, 0.0, 1.5, 9.0]])
    g0 = ref.gdn_decay_gate(v, np.zeros(5), dt)
    g1 = ref.gdn_decay_gate(v, np.full(5, math.log(2.0)), dt)
    assert np.allclose(g1, 2.0 * g0, rtol=1e-15, atol=0)
    # g <= 0, the forget gate exp(g) lies in (0, 1], and g falls as v grows
    vs = np.linspace(-20, 20, 81)[:, None]
    g = ref.gdn_decay_gate(vs, np.full(5, 1.3), dt)
    assert np.all(g < 0) and np.all(np.exp(g) <= 1.0) and np.all(np.exp(g) > 0)
    assert np.all(np.diff(g, axis=0) < 0)
    # far above zero, softplus(z) = z: g = -exp(A_log) (v + dt_bias)
    big = np.full((1, 5), 60.0)
    assert np.allclose(ref.gdn_decay_gate(big, np.full(5, 0.5), dt), -math.exp(0.5) * (60.0 + dt), rtol=1e-14)
    assert np.array_equal(ref.gdn_write_gate(v), ref.sigmoid(v))


def test_segmented_gates_are_the_segmented_gemm_then_the_gate_functions():
    rng = np.random.default_rng(5)
    rows = [24, 16, 8, 8]
    K = 64
    a = ref.quantize(rng.standard_normal((5, K)).astype(np.float32))
    ws = [ref.quantize((rng.standard_normal((r, K)) * 0.3).astype(np.float32)) for r in rows]
    wc = np.concatenate([w[0] for w in ws])
    wsc = np.concatenate([w[1] for w in ws])
    gs = [w[2] for w in ws]
    a_log = rng.uniform(0, 2.7, 8)
    dt_bias = rng.uniform(-6, -2, 8)
    Y, S = ref.gemm_segmented_ref(*a, wc, wsc, gs, rows)
    G, Y2, S2 = ref.gemm_segmented_gates_ref(*a, wc, wsc, gs, rows, 2, a_log, dt_bias, 3)
    assert np.array_equal(Y, Y2) and np.array_equal(S, S2)
    assert np.array_equal(G[:, :40], Y[:, :40])
    assert np.array_equal(G[:, 40:48], ref.gdn_decay_gate(Y[:, 40:48], a_log, dt_bias))
    assert np.array_equal(G[:, 48:], ref.sigmoid(Y[:, 48:]))
    G0, _, _ = ref.gemm_segmented_gates_ref(*a, wc, wsc, gs, rows, -1, None, None, -1)
    assert np.array_equal(G0, Y)
    # the decay module may come first and the write module before it
    G3, _, _ = ref.gemm_segmented_gates_ref(*a, wc, wsc, gs, rows, 0, rng.uniform(0, 1, 24), np.zeros(24), 1)
    assert np.all(G3[:, :24] < 0) and np.all((G3[:, 24:40] > 0) & (G3[:, 24:40] < 1))


def test_silu_identities_and_swiglu_composition():
    import math
    z = np.linspace(-40.0, 40.0, 321)
    assert ref.silu(0.0) == 0.0
    assert np.allclose(ref.silu(z) - ref.silu(-z), z, rtol=0, atol=1e-12)       # z (s(z) + s(-z)) = z
    assert abs(ref.silu(math.log(3.0)) - 0.75 * math.log(3.0)) < 1e-15
    assert abs(ref.silu(40.0) - 40.0) < 1e-15 and abs(ref.silu(-40.0)) < 1e-15
    h = 1e-6
    d = (ref.silu(z + h) - ref.silu(z - h)) / (2 * h)
    assert np.all(d <= 1.1) and np.all(d >= -0.1)                                  # the slope bound tests use
    rng = np.random.default_rng(9)
    a = ref.quantize(rng.standard_normal((3, 64)).astype(np.float32))
    w = ref.quantize((rng.standard_normal((2 * 32, 64)) * 0.2).astype(np.float32))
    H, G, U, SG, SU = ref.gemm_swiglu_ref(*a, *w)
    Y, S = ref.gemm_ref(*a, *w)
    assert np.array_equal(G, Y[:, :32]) and np.array_equal(U, Y[:, 32:]) and np.array_equal(SU, S[:, 32:])
    assert np.allclose(H, G / (1 + np.exp(-G)) * U, rtol=1e-13, atol=1e-300)
