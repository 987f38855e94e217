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
// One thread per scale byte.  The quotient is decided exactly in fp64:
// E4M3(s) g_i has at most 28 significant bits and every E4M3 midpoint times
// g* at most 29, so both sides of each comparison are exact doubles.  This
// is an offline transform over a few MB of scales, so no fast path is kept.
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

struct ModuleTable {
  int64_t row_end[kMaxModules];  // exclusive prefix sums of module row counts
  int32_t n;
};

__device__ __forceinline__ double e4m3_f64(uint32_t c) { return (double)e4m3_to_f32(c); }

__global__ void clear_counters_kernel(uint32_t* counters) {
  if (threadIdx.x < 2) counters[threadIdx.x] = 0u;
}

__global__ __launch_bounds__(256) void harmonize_kernel(uint8_t* __restrict__ scales,
                                                        const float* __restrict__ module_gs,
                                                        ModuleTable tab, int64_t scales_per_row,
                                                        float* __restrict__ shared_gs,
                                                        uint32_t* __restrict__ counters) {
  float gmax = module_gs[0];
  for (int i = 1; i < tab.n; ++i) gmax = fmaxf(gmax, module_gs[i]);
  const double gstar = (double)gmax;
  const int64_t total = tab.row_end[tab.n - 1] * scales_per_row;

  uint32_t n_inexact = 0, n_sub = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int64_t row = idx / scales_per_row;
    int m = 0;
    while (row >= tab.row_end[m]) ++m;
    const uint32_t s = scales[idx];
    const double target = e4m3_f64(s) * (double)module_gs[m];  // exact
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
    scales[idx] = (uint8_t)c;
    n_inexact += (e4m3_f64(c) * gstar != target) ? 1u : 0u;
    n_sub += (s != 0u && (c >> 3) == 0u) ? 1u : 0u;
  }
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
  int64_t acc = 0;
  for (int i = 0; i < n_modules; ++i) {
    acc += module_rows[i];
    tab.row_end[i] = acc;
  }
  tab.n = n_modules;
  const int64_t spr = K / 16;
  const int64_t total = acc * spr;
  if (counters) clear_counters_kernel<<<1, 64, 0, stream>>>(counters);
  int64_t grid = (total + 255) / 256;
  if (grid > 4096) grid = 4096;
  if (grid < 1) grid = 1;
  harmonize_kernel<<<(unsigned)grid, 256, 0, stream>>>(scales, module_gs, tab, spr, shared_gs, counters);
  return hipGetLastError();
}

}  // namespace nvfp4
