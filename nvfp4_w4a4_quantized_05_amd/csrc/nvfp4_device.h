// Device-side helpers shared by the NVFP4 kernels (gfx950 / CDNA4).
//
// Format recap (picx.dev summary of arXiv 2609.04098, "Background", item 1):
// E2M1 values {0, .5, 1, 1.5, 2, 3, 4, 6} with a sign bit, one E4M3 scale per
// 16 values (blockmax / 6), one FP32 scale per tensor.  Dequantized values
// are E2M1 x E4M3 products: at most 6 significant bits between 2^-10 and
// 2688, which fp16 represents exactly (normal range 2^-14 .. 65504).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBlock = 16;          // values per E4M3 block scale
constexpr float kE4M3Max = 448.0f;  // largest finite E4M3 (0x7E)
constexpr float kGlobalDiv = 2688.0f;  // 6 * 448

// E4M3 ("fn") byte -> fp32, exact (hardware conversion; subnormals kept).
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

// fp32 -> E4M3 byte, round-to-nearest-even.  Callers clamp to [0, 448]
// first: the hardware returns NaN (0x7F) for values rounding past 448.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xFFu;
}

// Tensor scale from the absolute maximum: RN32(amax / 2688), 1.0 if zero.
// HIP's float division is correctly rounded (IEEE) by default.
__device__ __forceinline__ float tensor_scale_from_amax(float amax) {
  float g = amax / kGlobalDiv;
  return g == 0.0f ? 1.0f : g;
}

}  // namespace nvfp4
