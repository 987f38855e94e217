// Fused-projection tensor-scale harmonization for gfx950.
//
// Modules of a fused projection (a GDN in-projection's qkv, z, a and b, each
// quantized with its own FP32 tensor scale g_i) are concatenated along N and
// served by one GEMM that can apply only one tensor scale.  cctest.ai, "Why
// Gated DeltaNet Holds Up Under 4-Bit Quantization", "Main findings", last
// bullet: this creates a global-scale mismatch and the released checkpoint
// is pre-harmonized; anthology record LIT-800, "Standing in the anthology":
// unrepaired, the decay and write gates were computed with mis-scaled
// weights.  The procedure is not on the pages.  Implemented here:
// g* = max_i g_i (no rescaled scale can then leave the E4M3 range), and each
// block scale s of module i becomes E4M3_RNE(E4M3(s) g_i / g*), exact real
// quotient; codes are not touched.
//
// The new scale depends only on the old scale byte and the module, so each
// workgroup first builds a table of all 256 byte values for every module
// (in LDS, with the exact decision below), then streams the scale bytes
// through it, 16 bytes per lane where the buffer is 16-byte aligned.  The
// quotient is decided exactly in fp64: E4M3(s) g_i has at most 28
// significant bits and every E4M3 midpoint times g* at most 29, so both
// sides of each comparison are exact doubles.
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

struct ModuleTable {
  int64_t byte_end[kMaxModules];  // prefix sums of module row counts times the scales per row
  int32_t n;
};

__device__ __forceinline__ double e4m3_f64(uint32_t c) { return (double)e4m3_to_f32(c); }

__global__ void clear_counters_kernel(uint32_t* counters) {
  if (threadIdx.x < 2) counters[threadIdx.x] = 0u;
}

// Table entry of scale byte s in a module with tensor scale gi: the new
// byte in bits 0-7, bit 8 set if E4M3(new) g* differs from E4M3(s) gi,
// bit 9 set if a nonzero s became a subnormal (or zero) scale.
__device__ uint32_t harmonized_entry(uint32_t s, double gi, double gstar) {
  const double target = e4m3_f64(s) * gi;  // exact
  // candidate by hardware RNE of the (rounded) quotient, then exact fix-up
  const float q = fminf((float)(target / gstar), kE4M3Max);
  uint32_t c = f32_to_e4m3(q);
  if (c > 0) {
    const double lo = 0.5 * (e4m3_f64(c - 1) + e4m3_f64(c)) * gstar;  // exact
    if (target < lo || (target == lo && (c & 1u))) c -= 1;
  }
  if (c < 0x7Eu) {
    const double hi = 0.5 * (e4m3_f64(c) + e4m3_f64(c + 1)) * gstar;
    if (target > hi || (target == hi && (c & 1u))) c += 1;
  }
  const uint32_t inexact = (e4m3_f64(c) * gstar != target) ? 1u : 0u;
  const uint32_t sub = (s != 0u && (c >> 3) == 0u) ? 1u : 0u;
  return c | (inexact << 8) | (sub << 9);
}

// Module of scale byte idx (idx below the last end): no division.
__device__ __forceinline__ int module_of(const ModuleTable& tab, int64_t idx) {
  int m = 0;
  while (idx >= tab.byte_end[m]) ++m;
  return m;
}

__global__ __launch_bounds__(256) void harmonize_kernel(uint8_t* __restrict__ scales,
                                                        const float* __restrict__ module_gs,
                                                        ModuleTable tab,
                                                        float* __restrict__ shared_gs,
                                                        uint32_t* __restrict__ counters) {
  __shared__ uint16_t lut[kMaxModules * 256];
  float gmax = module_gs[0];
  for (int i = 1; i < tab.n; ++i) gmax = fmaxf(gmax, module_gs[i]);
  const double gstar = (double)gmax;
  for (int e = threadIdx.x; e < tab.n * 256; e += blockDim.x)
    lut[e] = (uint16_t)harmonized_entry((uint32_t)(e & 255), (double)module_gs[e >> 8], gstar);
  __syncthreads();

  const int64_t total = tab.byte_end[tab.n - 1];
  uint32_t n_inexact = 0, n_sub = 0;
  auto map = [&](uint32_t byte, int m) -> uint32_t {
    const uint32_t v = lut[m * 256 + byte];
    n_inexact += (v >> 8) & 1u;
    n_sub += v >> 9;
    return v & 0xFFu;
  };
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  // 16-byte chunks when the buffer allows it (the tail and any misaligned
  // buffer go byte by byte); a chunk inside one module uses one table row
  const int64_t nchunks = ((uintptr_t)scales % 16 == 0) ? total / 16 : 0;
  for (int64_t ch = tid; ch < nchunks; ch += stride) {
    u32x4_t* p = reinterpret_cast<u32x4_t*>(scales) + ch;
    u32x4_t w = *p;
    const int m0 = module_of(tab, 16 * ch);
    const int m1 = module_of(tab, 16 * ch + 15);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t o = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int m = m0 == m1 ? m0 : module_of(tab, 16 * ch + 4 * d + k);
        o |= map((w[d] >> (8 * k)) & 0xFFu, m) << (8 * k);
      }
      w[d] = o;
    }
    *p = w;
  }
  for (int64_t idx = 16 * nchunks + tid; idx < total; idx += stride)
    scales[idx] = (uint8_t)map(scales[idx], module_of(tab, idx));
  if (counters) {
    for (int o = 32; o > 0; o >>= 1) {
      n_inexact += __shfl_xor(n_inexact, o, 64);
      n_sub += __shfl_xor(n_sub, o, 64);
    }
    if ((threadIdx.x & 63) == 0) {
      if (n_inexact) atomicAdd(&counters[0], n_inexact);
      if (n_sub) atomicAdd(&counters[1], n_sub);
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *shared_gs = gmax;
}

}  // namespace

hipError_t launch_harmonize(uint8_t* scales, const float* module_gs, const int64_t* module_rows,
                            int32_t n_modules, int64_t K, float* shared_gs, uint32_t* counters,
                            hipStream_t stream) {
  ModuleTable tab{};
  const int64_t spr = K / 16;
  int64_t acc = 0;
  for (int i = 0; i < n_modules; ++i) {
    acc += module_rows[i];
    tab.byte_end[i] = acc * spr;
  }
  tab.n = n_modules;
  const int64_t total = acc * spr;
  if (counters) clear_counters_kernel<<<1, 64, 0, stream>>>(counters);
  // one workgroup per CU at most: each builds the table once
  int64_t grid = (total / 16 + 255) / 256;
  if (grid > 256) grid = 256;
  if (grid < 1) grid = 1;
  harmonize_kernel<<<(unsigned)grid, 256, 0, stream>>>(scales, module_gs, tab, shared_gs, counters);
  return hipGetLastError();
}

}  // namespace nvfp4
