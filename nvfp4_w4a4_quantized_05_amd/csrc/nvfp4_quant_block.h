// One NVFP4 block: 16 values -> E4M3 scale byte + 16 packed E2M1 codes.
// Shared by the quantize kernel and the decode GEMM's fused activation
// quantization, so both produce the same bytes.
//
// What it computes (picx.dev summary of arXiv 2609.04098, "Background",
// item 1): an E4M3 scale equal to blockmax / 6 in units of the FP32 tensor
// scale g, and per value an E2M1 code, packed two per byte (even value in
// the low nibble).  Rounding is round-to-nearest-even of the exact real
// quotients blockmax / (6 g) and |x| / (scale g), saturated at 448 and 6.
//
// Exact rounding at fp32 cost.  The quotients are formed approximately in
// fp32 (a reciprocal and a multiply, a few ulp of error) and rounded by the
// hardware converters (fp8 for the scale, fp4 for the codes).  Where the
// approximate quotient could round differently from the exact one, the
// decision is taken exactly: with a value t exact in fp32 (a midpoint, or a
// grid value), fma(t * scale, g, -|x|) is the exact difference
// t*scale*g - |x| rounded once, so its sign, and whether it is zero (a tie),
// are exact.
//
//  * Block scale: both neighbouring midpoints of the converter's result are
//    checked that way (a few ops per block, no branch).
//  * Codes: every E2M1 decision point (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5)
//    has at most 2 mantissa bits, so between two consecutive values with at
//    most 2 mantissa bits, m1 < m2, the code is constant.  The exact
//    quotient q lies in [m1, m2] for the pair around it, and the approximate
//    quotient y rounded to 2 mantissa bits, m, is m1 or m2 (y is off by a few
//    ulp, far less than half the gap).  The exact sign of m*scale*g - |x|
//    says on which side of m the exact quotient lies (a zero: on m itself,
//    a tie if m is a decision point); m moved by 2^-8 of itself to that side
//    (on a tie, toward the even code) lies strictly inside q's interval, so
//    the converter's rounding of it is the exact-real code.  This holds for
//    every value, so every quotient takes the same few ops, with no test or
//    branch (grid values and values far from a decision point come out
//    unchanged in code).
#pragma once

#include "nvfp4_device.h"

namespace nvfp4 {
namespace {

// Exact E4M3 rounding of bm / (6 g) from the converter's result s0 for an
// approximate quotient: s0 - 1 if bm lies below the midpoint under s0 (or on
// it, with s0 odd), s0 + 1 if above the midpoint over s0 (or on it, with s0
// odd), else s0.  Sign tests on the bit patterns of the exact differences:
// (int)bits(d) + odd > 0 means d > 0, or d == +0 and s0 odd.
__device__ __forceinline__ uint32_t exact_scale(uint32_t s0, float v0, float bm, float g) {
  const uint32_t odd = s0 & 1u;
  // 6 x the midpoints below and above s0: 3 x (sum of two neighbouring E4M3
  // values), exact (at most 7 significant bits); NaN for s0 = 0 / 0x7E (unused)
  const float lo6 = 3.0f * (e4m3_to_f32(s0 - 1) + v0);
  const float hi6 = 3.0f * (v0 + e4m3_to_f32(s0 + 1));
  const int dl = (int)(__float_as_uint(fmaf(lo6, g, -bm)) + odd);  // > 0: round down
  const int du = (int)(__float_as_uint(fmaf(hi6, g, -bm)) - odd);  // < 0: round up
  uint32_t s = s0;
  s = (s0 > 0u && dl > 0) ? s0 - 1 : s;
  s = (s0 < 0x7Eu && du < 0) ? s0 + 1 : s;
  return s;
}

// Settled quotient for a value x with approximate quotient y: m = y rounded
// to 2 mantissa bits (ties away from zero), sign kept; with unit val(s) g:
// beyond m (|x| > |m| val(s) g) the result is m moved away from zero, short
// of it toward zero, and on a tie toward the even code: of the E2M1 decision
// points 0.25 | 0.75 | 1.25 | 1.75 | 2.5 | 3.5 | 5, exactly those with the
// first mantissa bit set (0.75, 1.75, 3.5) have an odd code below them.  So
// with d = the exact difference |m| val(s) g - |x| (never -0: the product is
// >= 0) and b = that mantissa bit of m, "round down" is d > 0, or d = +0
// and b = 0, i.e. (int)bits(d) >= b.  Moving m by 2^-8 of itself keeps its
// sign, which is y's (also for y = -0); m = +-0 stays +-0.
__device__ __forceinline__ float settle_e2m1(float y, float ax, float sval, float g) {
  const uint32_t mb = (__float_as_uint(y) + 0x100000u) & 0xFFE00000u;  // m, sign kept
  const float m = __uint_as_float(mb);
  const int b = (int)((mb >> 22) & 1u);
  const bool down = (int)__float_as_uint(fmaf(fabsf(m) * sval, g, -ax)) >= b;
  // a product, not m + m k: (1 -/+ 2^-8) m is exact (at most 12 significant
  // bits) and keeps the sign of m = -0
  return m * (down ? 1.0f - 0x1p-8f : 1.0f + 0x1p-8f);
}

// Quantize the 16 values v of one block with tensor scale g (r6 = approximate
// 1 / (6 g)): returns the E4M3 scale byte, codes in w0 (values 0-7) and w1
// (values 8-15), low nibble first.
__device__ __forceinline__ uint32_t quantize_block(const float v[16], float g, float r6, uint32_t& w0,
                                                   uint32_t& w1) {
  float bm = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) bm = fmaxf(bm, fabsf(v[i]));

  // block scale: RNE(bm / (6 g)) with saturation at 448
  const float q = fminf(bm * r6, kE4M3Max);
  const uint32_t s0 = f32_to_e4m3(q);
  const uint32_t s = exact_scale(s0, e4m3_to_f32(s0), bm, g);

  const float sval = e4m3_to_f32(s);
  const float rcp = s ? __builtin_amdgcn_rcpf(sval * g) : 0.0f;  // zero scale: all magnitudes 0

  float y[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) y[i] = settle_e2m1(v[i] * rcp, fabsf(v[i]), sval, g);
  w0 = 0;
  w1 = 0;
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, y[0], y[1], 1.0f, 0);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, y[2], y[3], 1.0f, 1);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, y[4], y[5], 1.0f, 2);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, y[6], y[7], 1.0f, 3);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, y[8], y[9], 1.0f, 0);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, y[10], y[11], 1.0f, 1);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, y[12], y[13], 1.0f, 2);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, y[14], y[15], 1.0f, 3);

  return s;
}

}  // namespace
}  // namespace nvfp4
