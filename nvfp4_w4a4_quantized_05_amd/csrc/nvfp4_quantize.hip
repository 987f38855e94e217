// NVFP4 activation/weight quantizer for gfx950.
//
// What it computes (picx.dev summary of arXiv 2609.04098, "Background",
// item 1): per 16-value block an E4M3 scale equal to blockmax / 6 (in units
// of the FP32 tensor scale g), and per value an E2M1 code, packed two per
// byte.  Rounding is round-to-nearest-even of the exact real quotients
// blockmax / (6 g) and |x| / (scale g), with saturation at 448 and 6.
//
// Design.  HBM-bound: 2.5625 bytes per bf16 value (2 in, 0.5 + 1/16 out).
// One lane owns one 16-value block: two 16-byte loads (bf16) or four (fp32),
// a block max in registers, one 8-byte code store and one scale byte.  A
// wave covers 64 consecutive blocks, so every load and store instruction of
// a wave touches one contiguous 1-2 KiB span.
//
// The per-block arithmetic (exact rounding at fp32 cost) is in
// nvfp4_quant_block.h.
#include "nvfp4_device.h"
#include "nvfp4_internal.h"
#include "nvfp4_quant_block.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
template <bool kBf16>
__device__ __forceinline__ void load_block(const void* base, int64_t elem_off, float v[16]) {
  if constexpr (kBf16) {
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(base) + elem_off);
    const u32x4_t a = __builtin_nontemporal_load(p);
    const u32x4_t b = __builtin_nontemporal_load(p + 1);
    const uint32_t w[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const floatx4_t* p = reinterpret_cast<const floatx4_t*>(reinterpret_cast<const float*>(base) + elem_off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const floatx4_t t = __builtin_nontemporal_load(p + i);
      v[4 * i] = t[0]; v[4 * i + 1] = t[1]; v[4 * i + 2] = t[2]; v[4 * i + 3] = t[3];
    }
  }
}

// kMode: 0 = tensor scale given in *gptr; 1 = *gptr holds amax bits (the
// finalize kernel turns it into g afterwards).
template <bool kBf16, bool kContig, int kMode>
__global__ __launch_bounds__(kThreads) void quantize_kernel(
    const void* __restrict__ x, int64_t nblocks, int64_t blocks_per_row, int64_t ldx,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, const float* __restrict__ gptr) {
  const float gin = *gptr;
  const float g = kMode == 1 ? tensor_scale_from_amax(gin) : gin;
  const float r6 = __builtin_amdgcn_rcpf(6.0f * g);  // approximate 1/(6g)

  const int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (b >= nblocks) return;
  int64_t off;
  if constexpr (kContig) {
    off = b * kBlock;
  } else {
    const int64_t row = b / blocks_per_row;
    off = row * ldx + (b - row * blocks_per_row) * kBlock;
  }
  float v[16];
  load_block<kBf16>(x, off, v);

  uint32_t w0, w1;
  const uint32_t s = quantize_block(v, g, r6, w0, w1);
  u32x2_t out;
  out[0] = w0;
  out[1] = w1;
  __builtin_nontemporal_store(out, reinterpret_cast<u32x2_t*>(codes) + b);
  // streaming stores for both (plain code stores measured 3-4% slower,
  // plain scale stores 1-2% slower)
  __builtin_nontemporal_store((uint8_t)s, scales + b);
}

// 16-byte chunk c of the tensor (8 bf16 or 4 fp32 values; chunks_per_row
// per row of ldx values).
template <bool kBf16, bool kContig>
__device__ __forceinline__ u32x4_t amax_chunk(const void* x, int64_t c, int64_t chunks_per_row, int64_t ldx) {
  constexpr int kPer = kBf16 ? 8 : 4;  // values per 16-byte chunk
  int64_t off;
  if constexpr (kContig) {
    off = c * kPer;
  } else {
    const int64_t row = c / chunks_per_row;
    off = row * ldx + (c - row * chunks_per_row) * kPer;
  }
  const int64_t byte_off = off * (kBf16 ? 2 : 4);
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint8_t*>(x) + byte_off));
}

template <bool kBf16>
__device__ __forceinline__ float amax_fold(float m, u32x4_t t) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (kBf16) {
      m = fmaxf(m, fabsf(__uint_as_float(t[i] << 16)));
      m = fmaxf(m, fabsf(__uint_as_float(t[i] & 0xFFFF0000u)));
    } else {
      m = fmaxf(m, fabsf(__uint_as_float(t[i])));
    }
  }
  return m;
}

constexpr int kAmaxUnroll = 4;
// At most 1024 workgroups (4 per CU), each streaming many windows: on the
// layer inputs (32768 x 4096 .. 17408 bf16) this read 5.6-6.8 TB/s, against
// 4.2-6.7 with 4096 workgroups and 5.3-6.8 with 512 x 8 or 1024 x 2 chunks
// per lane per pass.
constexpr int64_t kAmaxMaxGroups = 1024;

// Absolute maximum of the tensor into *amax_bits (float bits; all values
// non-negative, so unsigned max == float max).  *amax_bits starts at 0.
// Each pass of a workgroup reads one contiguous window of kAmaxUnroll x
// kThreads chunks (lane l: chunks l, l + kThreads, ...), all loads issued
// before the first max, so every lane keeps kAmaxUnroll loads in flight;
// the windows stride over the tensor by the grid.  The
// workgroup's maximum goes to *amax_bits with one atomic, and only if it
// exceeds the value already there (read first; the maximum only grows, so a
// skipped value is never the result): the atomics of all workgroups land on
// one address and queue there.  Against one atomic per workgroup and one
// chunk per lane per pass, this cut the amax pass from 75-95 us to 46-60 us
// on 32768 x {4096, 5120} bf16 inputs and from 194 to 170 us on 32768 x 17408.
template <bool kBf16, bool kContig>
__global__ __launch_bounds__(kThreads) void amax_kernel(const void* __restrict__ x, int64_t nchunks,
                                                        int64_t chunks_per_row, int64_t ldx,
                                                        uint32_t* __restrict__ amax_bits) {
  constexpr int64_t kWin = (int64_t)kAmaxUnroll * kThreads;
  float m = 0.0f;
  const int64_t step = (int64_t)gridDim.x * kWin;
  int64_t c = (int64_t)blockIdx.x * kWin + threadIdx.x;
  for (; c + (kAmaxUnroll - 1) * kThreads < nchunks; c += step) {
    u32x4_t t[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) t[u] = amax_chunk<kBf16, kContig>(x, c + u * kThreads, chunks_per_row, ldx);
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) m = amax_fold<kBf16>(m, t[u]);
  }
  // the last, partial window: this lane's chunks of it that exist
  for (; c < nchunks; c += kThreads) m = amax_fold<kBf16>(m, amax_chunk<kBf16, kContig>(x, c, chunks_per_row, ldx));
  // wave reduction, then one value per wave through LDS
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  __shared__ float part[kThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) part[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = part[0];
    for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, part[i]);
    const uint32_t rb = __float_as_uint(r);
    if (rb > __hip_atomic_load(amax_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
      atomicMax(amax_bits, rb);
  }
}

__global__ void clear_word_kernel(uint32_t* p) { *p = 0u; }

__global__ void finalize_scale_kernel(float* g) { *g = tensor_scale_from_amax(*g); }

template <bool kBf16, bool kContig>
hipError_t launch_typed(const void* x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* codes,
                        uint8_t* scales, float* gs, bool from_amax, hipStream_t stream) {
  const int64_t bpr = cols / kBlock;
  const int64_t nblocks = rows * bpr;
  if (from_amax) {
    clear_word_kernel<<<1, 1, 0, stream>>>(reinterpret_cast<uint32_t*>(gs));
    if (nblocks > 0) {  // no rows: the amax of no values is 0, so g = 1.0
      const int per = kBf16 ? 8 : 4;
      const int64_t cpr = cols / per;
      const int64_t nchunks = rows * cpr;
      int64_t grid = (nchunks + kThreads * kAmaxUnroll - 1) / (kThreads * kAmaxUnroll);
      if (grid > kAmaxMaxGroups) grid = kAmaxMaxGroups;
      if (grid < 1) grid = 1;
      amax_kernel<kBf16, kContig><<<(unsigned)grid, kThreads, 0, stream>>>(
          x, nchunks, cpr, ldx, reinterpret_cast<uint32_t*>(gs));
      quantize_kernel<kBf16, kContig, 1><<<(unsigned)((nblocks + kThreads - 1) / kThreads), kThreads, 0,
                                           stream>>>(x, nblocks, bpr, ldx, codes, scales, gs);
    }
    finalize_scale_kernel<<<1, 1, 0, stream>>>(gs);
  } else if (nblocks > 0) {
    quantize_kernel<kBf16, kContig, 0><<<(unsigned)((nblocks + kThreads - 1) / kThreads), kThreads, 0,
                                         stream>>>(x, nblocks, bpr, ldx, codes, scales, gs);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const void* x, bool in_bf16, int64_t rows, int64_t cols, int64_t ldx,
                           uint8_t* codes, uint8_t* scales, float* global_scale, bool from_amax,
                           hipStream_t stream) {
  const bool contig = (ldx == cols);
  if (in_bf16) {
    return contig ? launch_typed<true, true>(x, rows, cols, ldx, codes, scales, global_scale, from_amax, stream)
                  : launch_typed<true, false>(x, rows, cols, ldx, codes, scales, global_scale, from_amax, stream);
  }
  return contig ? launch_typed<false, true>(x, rows, cols, ldx, codes, scales, global_scale, from_amax, stream)
                : launch_typed<false, false>(x, rows, cols, ldx, codes, scales, global_scale, from_amax, stream);
}

}  // namespace nvfp4
