"""Exact-rational twin of the NVFP4 oracle, for brute-force checks on small inputs.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Written independently of ``nvfp4_ref``: values are ``fractions.Fraction``,
rounding scans the whole target grid for the nearest value (ties to the even
code), and nothing is vectorised.  It follows the same definition ([PX],
"Background", item 1: E2M1 values, an E4M3 scale of blockmax/6 per 16-element
block, one FP32 scale per tensor) so that agreement between the two pins the
fp64 implementation's exactness argument empirically.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction


def e2m1_magnitudes():
    """The 8 non-negative E2M1 values, indexed by the 3 magnitude bits."""
    vals = []
    for m in range(8):
        exp, man = m >> 1, m & 1
        if exp == 0:
            vals.append(Fraction(man, 2))
        else:
            vals.append((1 + Fraction(man, 2)) * Fraction(2) ** (exp - 1))
    return vals


def e4m3_values():
    """Values of E4M3 bytes 0..0x7E (0x7F is NaN in the fn variant)."""
    vals = []
    for c in range(0x7F):
        exp, man = c >> 3, c & 7
        if exp == 0:
            vals.append(Fraction(man, 8) * Fraction(2) ** -6)
        else:
            vals.append((1 + Fraction(man, 8)) * Fraction(2) ** (exp - 7))
    return vals


E2M1 = e2m1_magnitudes()
E4M3 = e4m3_values()


def nearest_even(q: Fraction, grid) -> int:
    """Index into the increasing grid of the value nearest q; ties to the even
    index; values past the end saturate to the last index."""
    if q >= grid[-1]:
        return len(grid) - 1
    best, best_d = 0, abs(q - grid[0])
    for i in range(1, len(grid)):
        d = abs(q - grid[i])
        if d < best_d or (d == best_d and i % 2 == 0):
            best, best_d = i, d
    return best


def to_fraction(v: float) -> Fraction:
    return Fraction(v)


def round_to_f32(q: Fraction) -> float:
    """Round a non-negative rational to the nearest IEEE binary32, ties to even
    (normals and subnormals; overflow is not needed here)."""
    if q == 0:
        return 0.0
    if q < 0:
        return -round_to_f32(-q)
    e = math.floor(math.log2(q.numerator) - math.log2(q.denominator))
    # fix up the estimate so that 2^e <= q < 2^(e+1)
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    e = max(e, -126)                    # subnormal range shares the 2^-149 quantum
    quantum = Fraction(2) ** (e - 23)
    n = q / quantum
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = Fraction(fl) * quantum
    out = struct.unpack("<f", struct.pack("<f", float(val)))[0]
    assert Fraction(out) == val
    return out


def global_scale_exact(values) -> float:
    amax = max((abs(Fraction(v)) for v in values), default=Fraction(0))
    g = round_to_f32(amax / 2688)
    return 1.0 if g == 0 else g


def quantize_block_exact(block, g: float):
    """(scale byte, [16 codes]) of one 16-element block under tensor scale g."""
    assert len(block) == 16
    gq = Fraction(g)
    bm = max(abs(Fraction(v)) for v in block)
    s = nearest_even(bm / (6 * gq), E4M3)
    unit = E4M3[s] * gq
    codes = []
    for v in block:
        sign = 8 if math.copysign(1.0, v) < 0 else 0
        if unit == 0:
            codes.append(sign)
        else:
            codes.append(sign | nearest_even(abs(Fraction(v)) / unit, E2M1))
    return s, codes


def dequant_exact(code: int, scale: int, g: float) -> Fraction:
    mag = E2M1[code & 7] * E4M3[scale] * Fraction(g)
    return -mag if code & 8 else mag


def gemm_exact(a_codes, a_scales, g_a, w_codes, w_scales, g_w):
    """Exact Y[m][n] = sum_k deqA[m][k] deqW[n][k] from unpacked code lists.

    a_codes: M lists of K codes; a_scales: M lists of K/16 scale bytes; same
    for W with N rows.  Returns a list of lists of Fractions.
    """
    M, N, K = len(a_codes), len(w_codes), len(a_codes[0])
    out = []
    for m in range(M):
        row = []
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += dequant_exact(a_codes[m][k], a_scales[m][k // 16], g_a) * \
                       dequant_exact(w_codes[n][k], w_scales[n][k // 16], g_w)
            row.append(acc)
        out.append(row)
    return out


def harmonize_scale_exact(scale: int, g_i: float, g_star: float) -> int:
    return nearest_even(E4M3[scale] * Fraction(g_i) / Fraction(g_star), E4M3)
