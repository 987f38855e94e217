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
// hardware converters (fp8 for the scale, fp4 for the codes).  That gives
// the exact-real answer unless the quotient lies within a few ulp of a
// rounding midpoint, where the decision is taken exactly: with the midpoint
// t (exact in fp32), fma(t * scale, g, -|x|) is the exact difference
// t*scale*g - |x| rounded once, so its sign, and whether it is zero (a tie),
// are exact.
//
//  * Block scale: both neighbouring midpoints of the converter's result are
//    checked that way, always (a few ops per block, no branch).
//  * Codes: every midpoint of the E2M1 grid has at most 2 mantissa bits, so
//    "near a midpoint" is read off the low mantissa bits of the approximate
//    quotient (grid points and zeros pass the test too, harmlessly).  When
//    any value of the wave's blocks is near, each flagged quotient y is
//    replaced by the nearby 2-mantissa-bit value m moved by 2^-8 of itself
//    toward the side the exact test gives (on a tie, toward the even code),
//    and the converter rounds that.  The move is far smaller than the gap
//    from m to any other decision point, so flagged grid values keep their
//    codes.  Generic fp32 data is near for about one value in 10^5; bf16
//    data far more often (its block maxima share short mantissas with the
//    tensor maximum, so quotients land on grid points and midpoints), which
//    is why both paths stay in vector registers, without per-value branches.
#pragma once

#include "nvfp4_device.h"

namespace nvfp4 {
namespace {

constexpr uint32_t kNearUlps = 16;  // margin (in ulps) of the near-midpoint test

// Exact E4M3 rounding of bm / (6 g) from the converter's result s0 for an
// approximate quotient: s0 - 1 if bm lies below the midpoint under s0 (or on
// it, with s0 odd), s0 + 1 if above the midpoint over s0 (or on it, with s0
// odd), else s0.  Sign tests on the bit patterns of the exact differences:
// (int)bits(d) + odd > 0 means d > 0, or d == +0 and s0 odd.
__device__ __forceinline__ uint32_t exact_scale(uint32_t s0, float v0, float bm, float g) {
  const uint32_t odd = s0 & 1u;
  const float lo = 0.5f * (e4m3_to_f32(s0 - 1) + v0);  // exact; NaN for s0 = 0 (unused)
  const float hi = 0.5f * (v0 + e4m3_to_f32(s0 + 1));  // exact; NaN for s0 = 0x7E (unused)
  const int dl = (int)(__float_as_uint(fmaf(lo * 6.0f, g, -bm)) + odd);  // > 0: round down
  const int du = (int)(__float_as_uint(fmaf(hi * 6.0f, g, -bm)) - odd);  // < 0: round up
  uint32_t s = s0;
  s = (s0 > 0u && dl > 0) ? s0 - 1 : s;
  s = (s0 < 0x7Eu && du < 0) ? s0 + 1 : s;
  return s;
}

// Near-midpoint key of a quotient's bit pattern b: <= 2 * kNearUlps when b
// is within kNearUlps ulps of a value with at most 2 mantissa bits.
__device__ __forceinline__ uint32_t e2m1_near_key(uint32_t b) { return (b + kNearUlps) & 0x1FFFFFu; }

// Settled quotient for a value x whose approximate quotient y lies next to a
// value with <= 2 mantissa bits, m.  With unit val(s) g: beyond m
// (|x| > |m| val(s) g) the result is |m| moved away from zero, short of it
// toward zero, and on a tie toward the even code: of the E2M1 decision
// points 0.25 | 0.75 | 1.25 | 1.75 | 2.5 | 3.5 | 5, exactly those with the
// first mantissa bit set (0.75, 1.75, 3.5) have an odd code below them.  The
// sign is y's (also for y = -0).
__device__ __forceinline__ float settle_e2m1(float y, float ax, float sval, float g) {
  const uint32_t mb = (__float_as_uint(y) + 0x100000u) & 0x7FE00000u;  // |m|
  const float m = __uint_as_float(mb);
  const uint32_t even_down = ((mb >> 22) & 1u) ^ 1u;
  const int d = (int)(__float_as_uint(fmaf(m * sval, g, -ax)) | even_down);  // > 0: round down
  const float r = fmaf(m, d > 0 ? -0x1p-8f : 0x1p-8f, m);
  return __uint_as_float((__float_as_uint(r) & 0x7FFFFFFFu) | (__float_as_uint(y) & 0x80000000u));
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
  uint32_t key = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    y[i] = v[i] * rcp;
    key = min(key, e2m1_near_key(__float_as_uint(y[i])));
  }
  if (key <= 2 * kNearUlps) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float ys = settle_e2m1(y[i], fabsf(v[i]), sval, g);
      y[i] = e2m1_near_key(__float_as_uint(y[i])) <= 2 * kNearUlps ? ys : y[i];
    }
  }
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
