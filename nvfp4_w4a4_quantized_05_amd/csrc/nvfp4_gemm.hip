// NVFP4 W4A4 GEMM for gfx950: y = RN32(g_a g_w) * deq(A) deq(W)^T.
//
// A = [M x K] and W = [N x K] are NVFP4 (picx.dev summary of arXiv
// 2609.04098, "Background", item 1: E2M1 codes two per byte, one E4M3 scale
// per 16 values along K, one FP32 scale per tensor).  The pages run this
// product on Blackwell's 4-bit tensor cores; that kernel design is not
// carried over.  On CDNA4 the 4-bit matrix instructions take power-of-two
// (E8M0) scales per 32 values, which cannot carry an E4M3 mantissa or a
// 16-value block, so the product is formed this way instead:
//
//  * Every dequantized value E2M1 x E4M3 has at most 6 significant bits in
//    [2^-10, 2688], so it is EXACT in fp16, and every product of two of them
//    is exact in fp32: the fp16 matrix instructions with fp32 accumulation
//    compute the same sum as the fp64 definition up to fp32 accumulation
//    rounding.  fp16 and bf16 matrix throughput is the same on gfx950; fp16
//    is used because gfx950 has a packed fp16 multiply and no packed bf16 one.
//  * Packed codes and scale bytes are staged through LDS (4.5 bits per value,
//    a quarter of the bytes an fp16 tile would need) and every wave
//    dequantizes its own operand fragments in registers: per 8 values one
//    hardware FP4->fp16 conversion per byte (with the exponent-only scale
//    2^8) and one packed fp16 multiply per pair by the block scale taken as
//    fp16 bits (scale byte << 7 = E4M3 value * 2^-8).  Both steps are exact.
//  * v_mfma_f32_32x32x16_f16: a lane supplies 8 consecutive K values of one
//    row.  Within an MFMA the K order is free as long as A and W agree, so a
//    lane of half h reads 32 contiguous code bytes (64 K values) of its row
//    from LDS and feeds them to 8 consecutive MFMAs; the 8 values of one MFMA
//    always sit inside one 16-value block, i.e. one scale.
//  * The RN32(g_a g_w) multiply and the fp32 or bf16 (RNE) conversion happen
//    in the epilogue, straight from the accumulators.
#include <cstdint>
#include <type_traits>

#include "nvfp4_device.h"
#include "nvfp4_internal.h"
#include "nvfp4_quant_block.h"

namespace nvfp4 {
namespace {

constexpr int kBK = 128;              // K values per main-loop step
constexpr int kRowBytes = kBK / 2;    // 64 code bytes per row per step
constexpr int kLdsRow = kRowBytes + 16;  // padded LDS row stride: conflict-free 16-byte reads
constexpr int kScaleBytes = kBK / 16;    // 8 scale bytes per row per step
constexpr size_t kDecodeMaxLds = 160 * 1024;  // LDS per workgroup on gfx950
// Waves per decode workgroup; each takes a contiguous part of K.  Eight
// (two per SIMD, M <= 16 without spills) measured about 10% slower than four
// at N = 12288 / 12384, K = 5120: each wave then has 2-3 tiles, so the ring's
// fill and the wider reduction weigh more.
constexpr int kDecodeWaves = 4;
// In-kernel activation quantization of the decode kernel: at most this many
// rows, and K up to kFusedMaxK.  The kernel handles up to 4 rows; at 3 and 4
// the quantize ALU work outgrows the time the weight loads leave free, and a
// separate quantize launch is faster (measured at N = 12288 and 12384,
// K = 5120).
constexpr int kFusedRows = 2, kFusedMaxK = 8192;

// fp16 pair (v, v) of an E4M3 scale byte times 2^-8.
__device__ __forceinline__ uint32_t scale_pair(uint32_t byte) {
  return (byte << 7) | (byte << 23);
}

// 8 consecutive codes (one dword, low nibble first) -> 8 exact fp16 values.
__device__ __forceinline__ half8_t dequant8(uint32_t codes, uint32_t s2) {
  const half2_t sc = __builtin_bit_cast(half2_t, s2);
  const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 0) * sc;
  const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 1) * sc;
  const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 2) * sc;
  const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 3) * sc;
  half8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Marks MFMA operands as still in use at this point of the program, so the
// register allocator cannot hand their registers to a new value before it.
template <int A, int B>
__device__ __forceinline__ void keep_live(const half8_t (&x)[A], const half8_t (&y)[B]) {
#pragma unroll
  for (int i = 0; i < A; ++i) __asm__ volatile("" ::"v"(x[i]));
#pragma unroll
  for (int i = 0; i < B; ++i) __asm__ volatile("" ::"v"(y[i]));
}

// Tile order: workgroups go round-robin to the 8 XCDs, so consecutive ids
// are first regrouped per XCD (each XCD's L2 then sees a compact range of
// tiles), and then walked in groups of kGroupM tile rows so that tiles in
// flight share A rows and W rows.
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int kXcd = 8, kGroupM = 8;
  const int ntiles = tiles_m * tiles_n;
  const int per = ntiles / kXcd, rem = ntiles % kXcd;
  const int x = bid % kXcd, i = bid / kXcd;
  const int t = (x < rem) ? x * (per + 1) + i : rem * (per + 1) + (x - rem) * per + i;
  const int group = kGroupM * tiles_n;
  const int first_m = (t / group) * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int r = t % group;
  tm = first_m + r % gsize;
  tn = r / gsize;
}

// Column range of `col` in the per-column tensor scales: the number of
// range ends at or below it (ends are non-decreasing).
__device__ __forceinline__ int col_range(const ColScales& cs, int col) {
  int s = 0;
  for (int i = 0; i + 1 < cs.n; ++i) s += col >= cs.end[i] ? 1 : 0;
  return s;
}

// RN32(g_a g_w) of output column `col`.
__device__ __forceinline__ float col_alpha(float g_a, const ColScales& cs, int col) {
  return g_a * cs.gs[col_range(cs, col)];
}

// silu(x) = x / (1 + e^-x) with the hardware exp2 of -x log2(e) and the
// hardware reciprocal: a few ulp, plus |x| 2^-23 relative from rounding
// x log2(e).  Large negative x gives 1 / inf = 0 (silu -> -0), large
// positive x gives x.
__device__ __forceinline__ float silu_fast(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}

// Whether output columns [c0, c1] meet a gate column range.
__device__ __forceinline__ bool cols_gated(const ColScales& cs, int c0, int c1) {
  return (c0 < cs.decay_hi && c1 >= cs.decay_lo) || (c0 < cs.write_hi && c1 >= cs.write_lo);
}

// Gate function of output column `col` applied to v = acc RN32(g_a g_w):
// the decay gate g = -exp(A_log) softplus(a + dt_bias) of the picx.dev
// summary page ("Introduction and Theoretical Foundation" > "Gated DeltaNet
// Mechanics") and the sigmoid write strength beta = sigmoid(b) (dmarx
// anthology record LIT-800, "Key takeaways", gates bullet).  fp32, with the
// device library's expf and log1pf; softplus(z) = max(z, 0) +
// log1p(exp(-|z|)) does not overflow.
__device__ __forceinline__ float col_gate(const ColScales& cs, int col, float v) {
  if (col >= cs.decay_lo && col < cs.decay_hi) {
    const int j = col - cs.decay_lo;
    const float z = v + cs.dt_bias[j];
    return -expf(cs.a_log[j]) * (fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z))));
  }
  if (col >= cs.write_lo && col < cs.write_hi) return 1.0f / (1.0f + expf(-v));
  return v;
}

template <bool kAligned>
__device__ __forceinline__ u32x4_t load_codes16(const uint8_t* row_ptr, int64_t byte_off, int64_t row_bytes,
                                               bool row_ok) {
  if (!row_ok) return u32x4_t{0, 0, 0, 0};
  if constexpr (kAligned) {
    return *reinterpret_cast<const u32x4_t*>(row_ptr + byte_off);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t v = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int64_t o = byte_off + 4 * d + b;
        if (o < row_bytes) v |= (uint32_t)row_ptr[o] << (8 * b);
      }
      w[d] = v;
    }
    return u32x4_t{w[0], w[1], w[2], w[3]};
  }
}

template <bool kAligned>
__device__ __forceinline__ u32x2_t load_scales8(const uint8_t* row_ptr, int64_t byte_off, int64_t row_bytes,
                                               bool row_ok) {
  if (!row_ok) return u32x2_t{0, 0};
  if constexpr (kAligned) {
    return *reinterpret_cast<const u32x2_t*>(row_ptr + byte_off);
  } else {
    uint32_t w[2];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      uint32_t v = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int64_t o = byte_off + 4 * d + b;
        if (o < row_bytes) v |= (uint32_t)row_ptr[o] << (8 * b);
      }
      w[d] = v;
    }
    return u32x2_t{w[0], w[1]};
  }
}

// One workgroup computes a BM x BN tile with (BM/WM) x (BN/WN) waves, each
// wave a WM x WN sub-tile of 32x32 MFMA blocks.
template <int BM, int BN, int WM, int WN, bool kAligned, bool kOutBf16>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void gemm_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_gs,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, const ColScales cs,
    int M, int N, int K, void* __restrict__ y, int64_t ldy) {
  constexpr int kWavesM = BM / WM, kWavesN = BN / WN;
  constexpr int kThreads = kWavesM * kWavesN * 64;
  constexpr int FM = WM / 32, FN = WN / 32;  // MFMA blocks per wave
  static_assert(BM % WM == 0 && BN % WN == 0 && WM % 32 == 0 && WN % 32 == 0, "tile shape");
  static_assert((BM * 4) % kThreads == 0 && (BN * 4) % kThreads == 0, "code loads per thread");
  static_assert(BM <= kThreads && BN <= kThreads, "scale loads: one row per thread");
  constexpr int kACodeLoads = BM * 4 / kThreads;  // 16-byte code chunks per thread per step
  constexpr int kWCodeLoads = BN * 4 / kThreads;

  __shared__ __attribute__((aligned(16))) uint8_t a_lds[2][BM * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint8_t w_lds[2][BN * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint8_t as_lds[2][BM * kScaleBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ws_lds[2][BN * kScaleBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wave_m = wave / kWavesN, wave_n = wave % kWavesN;
  const int r32 = lane & 31, half = lane >> 5;

  int tile_m, tile_n;
  tile_coords(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tile_m, tile_n);
  const int m0 = tile_m * BM, n0 = tile_n * BN;

  const int64_t row_bytes = K / 2, srow_bytes = K / 16;
  const int ksteps = (K + kBK - 1) / kBK;

  // global -> register staging (next step), then register -> LDS
  u32x4_t a_stage[kACodeLoads], w_stage[kWCodeLoads];
  u32x2_t as_stage = {0, 0}, ws_stage = {0, 0};

  auto load_step = [&](int ks) {
    const int64_t kb = (int64_t)ks * kRowBytes;
#pragma unroll
    for (int i = 0; i < kACodeLoads; ++i) {
      const int row = i * (kThreads / 4) + tid / 4;
      const int gm = m0 + row;
      a_stage[i] = load_codes16<kAligned>(a_codes + (int64_t)gm * row_bytes, kb + (tid & 3) * 16, row_bytes, gm < M);
    }
#pragma unroll
    for (int i = 0; i < kWCodeLoads; ++i) {
      const int row = i * (kThreads / 4) + tid / 4;
      const int gn = n0 + row;
      w_stage[i] = load_codes16<kAligned>(w_codes + (int64_t)gn * row_bytes, kb + (tid & 3) * 16, row_bytes, gn < N);
    }
    const int64_t sb = (int64_t)ks * kScaleBytes;
    if (tid < BM) {
      const int gm = m0 + tid;
      as_stage = load_scales8<kAligned>(a_scales + (int64_t)gm * srow_bytes, sb, srow_bytes, gm < M);
    }
    if (tid < BN) {
      const int gn = n0 + tid;
      ws_stage = load_scales8<kAligned>(w_scales + (int64_t)gn * srow_bytes, sb, srow_bytes, gn < N);
    }
  };
  auto store_step = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kACodeLoads; ++i) {
      const int row = i * (kThreads / 4) + tid / 4;
      *reinterpret_cast<u32x4_t*>(&a_lds[buf][row * kLdsRow + (tid & 3) * 16]) = a_stage[i];
    }
#pragma unroll
    for (int i = 0; i < kWCodeLoads; ++i) {
      const int row = i * (kThreads / 4) + tid / 4;
      *reinterpret_cast<u32x4_t*>(&w_lds[buf][row * kLdsRow + (tid & 3) * 16]) = w_stage[i];
    }
    if (tid < BM) *reinterpret_cast<u32x2_t*>(&as_lds[buf][tid * kScaleBytes]) = as_stage;
    if (tid < BN) *reinterpret_cast<u32x2_t*>(&ws_lds[buf][tid * kScaleBytes]) = ws_stage;
  };

  floatx16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  load_step(0);
  store_step(0);
  __syncthreads();

  for (int ks = 0; ks < ksteps; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < ksteps) load_step(ks + 1);

    // this lane's 32 code bytes (64 K values) and 4 scales per fragment row
    u32x4_t a_raw[FM][2], w_raw[FN][2];
    uint32_t a_sc[FM], w_sc[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = wave_m * WM + i * 32 + r32;
      const uint8_t* p = &a_lds[buf][row * kLdsRow + half * 32];
      a_raw[i][0] = *reinterpret_cast<const u32x4_t*>(p);
      a_raw[i][1] = *reinterpret_cast<const u32x4_t*>(p + 16);
      a_sc[i] = *reinterpret_cast<const uint32_t*>(&as_lds[buf][row * kScaleBytes + half * 4]);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int row = wave_n * WN + j * 32 + r32;
      const uint8_t* p = &w_lds[buf][row * kLdsRow + half * 32];
      w_raw[j][0] = *reinterpret_cast<const u32x4_t*>(p);
      w_raw[j][1] = *reinterpret_cast<const u32x4_t*>(p + 16);
      w_sc[j] = *reinterpret_cast<const uint32_t*>(&ws_lds[buf][row * kScaleBytes + half * 4]);
    }

    // Software pipeline over the 8 MFMA k-steps of this K tile: the operands
    // of step kk+1 are dequantized (VALU) while the MFMAs of step kk run,
    // and the scheduler is asked to alternate one MFMA with a few VALU ops so
    // that in-order issue never parks the VALU work behind a queue of MFMAs.
    half8_t af[2][FM], wf[2][FN];
    auto dequant_step = [&](int kk, int slot) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[slot][i] = dequant8(a_raw[i][kk >> 2][kk & 3], scale_pair((a_sc[i] >> (8 * (kk >> 1))) & 0xFFu));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        wf[slot][j] = dequant8(w_raw[j][kk >> 2][kk & 3], scale_pair((w_sc[j] >> (8 * (kk >> 1))) & 0xFFu));
    };
    dequant_step(0, 0);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < 8) dequant_step(kk + 1, cur ^ 1);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[cur][i], wf[cur][j], acc[i][j], 0, 0, 0);
      if (kk + 1 < 8) {
        constexpr int kValuPerMfma = (8 * (FM + FN) + FN * FM - 1) / (FM * FN);
#pragma unroll
        for (int g = 0; g < FM * FN; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);   // then VALU
        }
      }
    }

    if (ks + 1 < ksteps) store_step(buf ^ 1);
    __syncthreads();
  }

  // epilogue: y = acc * RN32(g_a g_w) with the column's g_w (then the
  // column's gate function, if any)
  const float g_a = *a_gs;
  const bool gated = cols_gated(cs, n0, n0 + BN - 1);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wave_n * WN + j * 32 + r32;
      if (col >= N) continue;
      const float alpha = col_alpha(g_a, cs, col);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wave_m * WM + i * 32 + (v >> 2) * 8 + half * 4 + (v & 3);
        if (row < M) {
          float o = acc[i][j][v] * alpha;
          if (gated) o = col_gate(cs, col, o);
          if constexpr (kOutBf16) {
            reinterpret_cast<__bf16*>(y)[(int64_t)row * ldy + col] = (__bf16)o;
          } else {
            reinterpret_cast<float*>(y)[(int64_t)row * ldy + col] = o;
          }
        }
      }
    }
  }
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// Direct global -> LDS copies (no VGPR staging): each lane's bytes land at
// lds_base + lane * size, so one wave instruction fills a contiguous span.
__device__ __forceinline__ void lds_copy16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)g, (lds_void_t*)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void lds_copy4(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)g, (lds_void_t*)lds_base, 4, 0, 0);
}

// Buffer-resource variant: base and size in SGPRs, a 32-bit per-lane offset
// and a wave-uniform offset.  Offsets past the resource size read zeros.
constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferFlags);
}
__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_base, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void lds_copy4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_base, 4, voff, soff, 0, 0);
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// XOR swizzle of the four 16-byte chunks of a 64-byte LDS row: the 32 rows
// read by one fragment load then hit distinct bank groups in every 8- and
// 16-lane phase of ds_read_b128.
__device__ __forceinline__ int chunk_swizzle(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

// Streaming kernel for the large shapes (K % 128 == 0, aligned operands).
//
// * 256 x 256 output tile per workgroup, 4 waves of 128 x 128 (4 x 4 blocks
//   of 32 x 32), accumulators in AGPRs.
// * K tiles of 128 values stream through a STAGES-deep LDS ring filled by
//   direct global -> LDS copies (no VGPR staging), STAGES K tiles ahead.
// * Each K tile is consumed in two halves.  While the MFMAs of one half run,
//   the LDS reads for the next half are in flight, and the one barrier per
//   K tile sits between the halves: after it the slot just read can be
//   refilled and the next K tile's first half read.  No wait on LDS or on
//   memory is then exposed in steady state except the barrier itself.
// * The MFMA takes W as its "A" operand and A as "B", so each lane's
//   accumulators hold 4 consecutive output columns of one row: the epilogue
//   stages rows in LDS with 8-byte writes and stores 16-byte row chunks.
// Rows past M or N read a clamped (valid) row; their outputs are never stored.
template <int STAGES, bool kOutBf16, bool kGates, bool kSwiglu>
__global__ __launch_bounds__(256) void gemm_stream_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_gs,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, const ColScales cs,
    int M, int N, int K, void* __restrict__ y, int64_t ldy, const SwigluOut sw) {
  constexpr int BM = 256, BN = 256, WM = 128, WN = 128, FM = 4, FN = 4;
  constexpr int kCodeBytes = BM * kRowBytes;          // 16 KiB per operand per stage
  constexpr int kStageScaleBytes = BM * kScaleBytes;  // 2 KiB per operand per stage
  constexpr int kStageBytes = 2 * kCodeBytes + 2 * kStageScaleBytes;
  constexpr int kLoadsPerStage = 12;                  // vector-memory instructions per wave per stage
  using out_t = typename std::conditional<kOutBf16, __bf16, float>::type;
  constexpr int kEsz = sizeof(out_t);
  // Output staged per pass: a whole 32-row block (every lane then writes in
  // every pass) by 256 bytes of each row: all 128 columns of the wave for
  // bf16, half of them for fp32.
  constexpr int kStripRows = 32;
  constexpr int kColPasses = kOutBf16 ? 1 : 2;
  constexpr int kStripCols = WN / kColPasses;
  constexpr int kStripRow = kStripCols * kEsz + 16;   // staged row bytes (+16 against bank conflicts)
  constexpr int kStripBytes = kStripRows * kStripRow;
  static_assert(STAGES >= 3, "ring depth");
  static_assert((STAGES - 1) * kLoadsPerStage < 64, "vmcnt range");
  constexpr int kAlphaBytes = WN * 4;                 // per-wave column scale table
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * kStageBytes + 4 * kStripBytes + 4 * kAlphaBytes];
  uint8_t* const ring = smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int wave_m = wave >> 1, wave_n = wave & 1;
  const int r32 = lane & 31, half = lane >> 5;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int64_t row_bytes = K / 2, srow_bytes = K / 16;
  const int ksteps = K / kBK;
  const bool vec_ok = ((uintptr_t)y % 16 == 0) && ((ldy * kEsz) % 16 == 0);

  // Per-lane copy offsets of the current tile (32-bit, within buffer
  // resources whose size bounds every read).  Wave w copies rows
  // [64w, 64w+64) of both operands: codes with 4 instructions of 16 rows x 4
  // (swizzled) 16-byte chunks, scales with 2 instructions of 32 rows x 2
  // dwords.  Rows past the operand are clamped to its last row.
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_codes, (int64_t)M * row_bytes);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w_codes, (int64_t)N * row_bytes);
  const __amdgpu_buffer_rsrc_t ras = make_rsrc(a_scales, (int64_t)M * srow_bytes);
  const __amdgpu_buffer_rsrc_t rws = make_rsrc(w_scales, (int64_t)N * srow_bytes);
  uint32_t a_off[4], w_off[4], as_off[2], ws_off[2];
  // W row of tile row r.  kSwiglu: the tile's 256 rows are gate and up rows
  // of its 128 output columns c0 = n0 / 2 .. + 127, in blocks of 32: wave
  // half wn = r / 128 covers columns c0 + 64 wn + 32 b + e (b = (r / 64) % 2,
  // e = r % 32), rows 32 b .. of the half being gate (r / 32 even) or up
  // (odd).  So a lane's accumulator blocks j = 0, 2 (gate) and 1, 3 (up) hold
  // the same output elements.  Rows past F repeat row F - 1 (outputs past F
  // are not written).
  auto w_row = [&](int n0, int r) -> int {
    if constexpr (kSwiglu) {
      const int col = n0 / 2 + 64 * (r >> 7) + 32 * ((r >> 6) & 1) + (r & 31);
      return min(col, sw.F - 1) + (((r >> 5) & 1) ? sw.F : 0);
    } else {
      return min(n0 + r, N - 1);
    }
  };
  auto set_sources = [&](int m0, int n0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wave * 64 + 16 * i + (lane >> 2);
      const int chunk = (lane & 3) ^ chunk_swizzle(row);
      a_off[i] = (uint32_t)min(m0 + row, M - 1) * (uint32_t)row_bytes + chunk * 16;
      w_off[i] = (uint32_t)w_row(n0, row) * (uint32_t)row_bytes + chunk * 16;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = wave * 64 + 32 * i + (lane >> 1);
      as_off[i] = (uint32_t)min(m0 + row, M - 1) * (uint32_t)srow_bytes + (lane & 1) * 4;
      ws_off[i] = (uint32_t)w_row(n0, row) * (uint32_t)srow_bytes + (lane & 1) * 4;
    }
  };
  auto issue_stage = [&](int ks, int slot) {
    uint8_t* st = ring + slot * kStageBytes;
    const uint32_t kc = (uint32_t)ks * kRowBytes, kscl = (uint32_t)ks * kScaleBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_copy16(ra, a_off[i], kc, st + (wave * 64 + 16 * i) * kRowBytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_copy16(rw, w_off[i], kc, st + kCodeBytes + (wave * 64 + 16 * i) * kRowBytes);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      lds_copy4(ras, as_off[i], kscl, st + 2 * kCodeBytes + (wave * 64 + 32 * i) * kScaleBytes);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      lds_copy4(rws, ws_off[i], kscl, st + 2 * kCodeBytes + kStageScaleBytes + (wave * 64 + 32 * i) * kScaleBytes);
  };

  // Fragment registers: raw[.][h] holds the 16 code bytes of K-tile half h
  // (MFMA steps 4h .. 4h+3); sc holds the 4 block scales of the K tile.
  u32x4_t a_raw[FM][2], w_raw[FN][2];
  uint32_t a_sc[FM], w_sc[FN], a_sc_next[FM], w_sc_next[FN];
  auto read_half = [&](int slot, int h, bool with_scales) {
    const uint8_t* st = ring + slot * kStageBytes;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = wave_m * WM + i * 32 + r32;
      a_raw[i][h] = *reinterpret_cast<const u32x4_t*>(st + row * kRowBytes + 16 * ((2 * half + h) ^ chunk_swizzle(row)));
      if (with_scales) a_sc_next[i] = *reinterpret_cast<const uint32_t*>(st + 2 * kCodeBytes + row * kScaleBytes + half * 4);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int row = wave_n * WN + j * 32 + r32;
      w_raw[j][h] = *reinterpret_cast<const u32x4_t*>(st + kCodeBytes + row * kRowBytes + 16 * ((2 * half + h) ^ chunk_swizzle(row)));
      if (with_scales)
        w_sc_next[j] = *reinterpret_cast<const uint32_t*>(st + 2 * kCodeBytes + kStageScaleBytes + row * kScaleBytes + half * 4);
    }
  };

  half8_t af[2][FM], wf[2][FN];
  auto dequant_step = [&](int kk, int slot) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
      af[slot][i] = dequant8(a_raw[i][kk >> 2][kk & 3], scale_pair((a_sc[i] >> (8 * (kk >> 1))) & 0xFFu));
#pragma unroll
    for (int j = 0; j < FN; ++j)
      wf[slot][j] = dequant8(w_raw[j][kk >> 2][kk & 3], scale_pair((w_sc[j] >> (8 * (kk >> 1))) & 0xFFu));
  };


  int tile_m, tile_n;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tile_m, tile_n);
  const int m0 = tile_m * BM, n0 = tile_n * BN;
  set_sources(m0, n0);
  // The ring always holds STAGES copies in flight or landed.  Past the last
  // K tile the copies repeat the last one into a slot nobody reads again,
  // which keeps the loop body free of branches (one scheduling region, so
  // copies and LDS reads can be interleaved with the matrix instructions).
#pragma unroll
  for (int s = 0; s < STAGES; ++s) issue_stage(min(s, ksteps - 1), s);

  floatx16_t acc[FN][FM];  // acc[j][i]: rows of W block j (output columns) x columns of A block i (output rows)
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.0f;
  // Main loop: a fixed software pipeline.  Each of the 8 MFMA steps of a K
  // tile issues its 16 MFMAs one at a time, each followed by one chunk of
  // the dequantization of the next step (about 4-7 VALU) and, in some steps,
  // one LDS read or one copy; a scheduling barrier after every group keeps
  // that order, so the dequantization runs in the shadow of the matrix
  // instructions instead of in blocks between them.  Step 7 dequantizes
  // step 0 of the next K tile (its half 0 and scales are read at mid-tile).
  //
  // Operand chunks follow the order in which the previous step last read
  // the operand's registers (W block j is last read by MFMA 4j + 3, A block
  // i by MFMA 12 + i): W0, W1, A0, A1, A2, A3, W2, W3.
  half2_t part[2];  // first half of an operand, between its two chunks
  auto dequant_chunk = [&](int t, int slot, int c, bool next_tile) {
    const int op = c >> 1, second = c & 1;
    constexpr int kOrder[8] = {4, 5, 0, 1, 2, 3, 6, 7};  // 0..3: A blocks, 4..7: W blocks
    const int o = kOrder[op];
    const bool is_w = o >= 4;
    const int idx = is_w ? o - 4 : o;
    const uint32_t sc = is_w ? (next_tile ? w_sc_next[idx] : w_sc[idx]) : (next_tile ? a_sc_next[idx] : a_sc[idx]);
    const uint32_t codes = is_w ? w_raw[idx][t >> 2][t & 3] : a_raw[idx][t >> 2][t & 3];
    const half2_t sp = __builtin_bit_cast(half2_t, scale_pair((sc >> (8 * (t >> 1))) & 0xFFu));
    if (!second) {
      part[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 0) * sp;
      part[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 1) * sp;
    } else {
      const half2_t q0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 2) * sp;
      const half2_t q1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 3) * sp;
      half8_t r;
      r[0] = part[0][0]; r[1] = part[0][1]; r[2] = part[1][0]; r[3] = part[1][1];
      r[4] = q0[0]; r[5] = q0[1]; r[6] = q1[0]; r[7] = q1[1];
      if (is_w) wf[slot][idx] = r;
      else af[slot][idx] = r;
    }
  };

  // first K tile: wait for its copies, read its first half + scales and
  // dequantize its step 0
  wait_vmcnt<(STAGES - 1) * kLoadsPerStage>();
  __builtin_amdgcn_s_barrier();
  read_half(0, 0, true);
#pragma unroll
  for (int i = 0; i < FM; ++i) a_sc[i] = a_sc_next[i];
#pragma unroll
  for (int j = 0; j < FN; ++j) w_sc[j] = w_sc_next[j];
  dequant_step(0, 0);

  // LDS reads of half h of a stage, one per call (g = 0..FM+FN-1 codes,
  // then FM+FN scale dwords when with_scales)
  auto read_one = [&](int slot, int h, int g) {
    const uint8_t* st = ring + slot * kStageBytes;
    if (g < FM) {
      const int row = wave_m * WM + g * 32 + r32;
      a_raw[g][h] = *reinterpret_cast<const u32x4_t*>(st + row * kRowBytes + 16 * ((2 * half + h) ^ chunk_swizzle(row)));
    } else if (g < FM + FN) {
      const int row = wave_n * WN + (g - FM) * 32 + r32;
      w_raw[g - FM][h] = *reinterpret_cast<const u32x4_t*>(st + kCodeBytes + row * kRowBytes + 16 * ((2 * half + h) ^ chunk_swizzle(row)));
    } else if (g < 2 * FM + FN) {
      const int row = wave_m * WM + (g - FM - FN) * 32 + r32;
      a_sc_next[g - FM - FN] = *reinterpret_cast<const uint32_t*>(st + 2 * kCodeBytes + row * kScaleBytes + half * 4);
    } else {
      const int row = wave_n * WN + (g - 2 * FM - FN) * 32 + r32;
      w_sc_next[g - 2 * FM - FN] =
          *reinterpret_cast<const uint32_t*>(st + 2 * kCodeBytes + kStageScaleBytes + row * kScaleBytes + half * 4);
    }
  };
  // the 12 copies of one stage, one per call
  auto issue_one = [&](int ks, int slot, int g) {
    uint8_t* st = ring + slot * kStageBytes;
    const uint32_t kc = (uint32_t)ks * kRowBytes, kscl = (uint32_t)ks * kScaleBytes;
    if (g < 4) lds_copy16(ra, a_off[g], kc, st + (wave * 64 + 16 * g) * kRowBytes);
    else if (g < 8) lds_copy16(rw, w_off[g - 4], kc, st + kCodeBytes + (wave * 64 + 16 * (g - 4)) * kRowBytes);
    else if (g < 10) lds_copy4(ras, as_off[g - 8], kscl, st + 2 * kCodeBytes + (wave * 64 + 32 * (g - 8)) * kScaleBytes);
    else lds_copy4(rws, ws_off[g - 10], kscl, st + 2 * kCodeBytes + kStageScaleBytes + (wave * 64 + 32 * (g - 10)) * kScaleBytes);
  };

  for (int ks = 0; ks < ksteps; ++ks) {
    const int slot = ks % STAGES, next_slot = (ks + 1) % STAGES;
    const int refill = min(ks + STAGES, ksteps - 1);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int cur = kk & 1;
      if (kk == 4) {
        // mid-tile: K tile ks+1 has landed (own copies + barrier), and every
        // wave is done reading this slot (its half 1 was read in step 0), so
        // the slot is refilled with K tile ks+STAGES (clamped).  A bare
        // s_barrier: __syncthreads() would also wait for every copy in
        // flight and drain the ring.
        wait_vmcnt<(STAGES - 2) * kLoadsPerStage>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int g = 0; g < FM * FN; ++g) {
        const int j = g >> 2, i = g & 3;
        acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[cur][j], af[cur][i], acc[j][i], 0, 0, 0);
        if (kk < 7) dequant_chunk(kk + 1, cur ^ 1, g, false);
        else dequant_chunk(0, 0, g, true);  // step 0 of the next K tile
        if (kk == 0 && g < FM + FN) read_one(slot, 1, g);  // half 1 of this K tile
        if (kk == 4 && g < kLoadsPerStage) issue_one(refill, slot, g);
        if (kk == 5) read_one(next_slot, 0, g);          // half 0 + scales of the next K tile
        __builtin_amdgcn_sched_barrier(0);
      }
      if (kk == 7) {
#pragma unroll
        for (int i = 0; i < FM; ++i) a_sc[i] = a_sc_next[i];
#pragma unroll
        for (int j = 0; j < FN; ++j) w_sc[j] = w_sc_next[j];
      }
    }
  }
  wait_vmcnt<0>();  // the repeated copies past the last K tile
  __syncthreads();  // every wave is done with the ring

  // Epilogue.  Lane (r32, half) of block (j, i) holds, for output row
  // m = m0 + 128 wave_m + 32 i + r32, the columns n0 + 128 wave_n + 32 j +
  // 8 (v / 4) + 4 half + (v % 4), v = 0..15: four consecutive columns per
  // group of 4 accumulators.  Rows go through LDS in strips of 32 rows by
  // 256 bytes (128 bf16 or 64 fp32 columns).  RN32(g_a g_w) of the wave's 128 columns goes to a
  // small LDS table, from which each lane reads the scales of its 64
  // columns once.  When one column range covers all 128 columns (every plain
  // GEMM, and most tiles of a segmented one) the table is filled with one
  // value, found with one lookup.
  const float g_a = *a_gs;
  if constexpr (kSwiglu) {
    // h = silu(g) u of the wave's 64 output columns c_out .. + 63 (v = acc
    // RN32(g_a g_w) for both), staged in fp32 in the wave's strip buffer, 32
    // rows at a time: 32 x 64 values, i.e. 128 blocks of 16, two per lane.
    // Each lane then quantizes its blocks with the quantize kernel's
    // arithmetic and stores 8 code bytes and 1 scale byte per block (and, if
    // asked, the 16 fp32 values).
    static_assert(kStripBytes >= 32 * 64 * 4, "fp32 strip of 32 x 64");
    const float alpha = g_a * cs.gs[0];
    const int c_out = n0 / 2 + 64 * wave_n;
    float* fs = reinterpret_cast<float*>(smem + STAGES * kStageBytes + wave * kStripBytes);
    const float hg = *sw.gs, r6 = __builtin_amdgcn_rcpf(6.0f * hg);
    const int qr = lane >> 2, qb = lane & 3;  // the lane's blocks: rows qr and 16 + qr, 16-column block qb
    if (c_out < sw.F) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        // the 32 rows of block i, every lane writing its values
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float gv = acc[2 * jj][i][v] * alpha, uv = acc[2 * jj + 1][i][v] * alpha;
            fs[r32 * 64 + 32 * jj + (v >> 2) * 8 + half * 4 + (v & 3)] = silu_fast(gv) * uv;
          }
        __asm__ volatile("" ::: "memory");  // other lanes' values are read below
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          const int row = m0 + wave_m * WM + i * 32 + sub * 16 + qr;
          const floatx4_t* src = reinterpret_cast<const floatx4_t*>(fs + (sub * 16 + qr) * 64 + 16 * qb);
          float vals[16];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const floatx4_t f4 = src[e];
#pragma unroll
            for (int t = 0; t < 4; ++t) vals[4 * e + t] = f4[t];
          }
          if (row < M) {
            uint32_t w0, w1;
            const uint32_t sc = quantize_block(vals, hg, r6, w0, w1);
            const int col = c_out + 16 * qb;
            *reinterpret_cast<u32x2_t*>(sw.codes + (int64_t)row * (sw.F / 2) + col / 2) = u32x2_t{w0, w1};
            sw.scales[(int64_t)row * (sw.F / 16) + col / 16] = (uint8_t)sc;
            if (sw.h) {
              floatx4_t* dst = reinterpret_cast<floatx4_t*>(sw.h + (int64_t)row * sw.ldh + col);
#pragma unroll
              for (int e = 0; e < 4; ++e) dst[e] = floatx4_t{vals[4 * e], vals[4 * e + 1], vals[4 * e + 2], vals[4 * e + 3]};
            }
          }
        }
        __asm__ volatile("" ::: "memory");  // reads done before the next block is written
      }
    }
    return;
  }
  const int c_first = n0 + wave_n * WN, c_last = min(c_first + WN, N) - 1;
  const int s_first = col_range(cs, c_first);
  float* const alpha_tab = reinterpret_cast<float*>(smem + STAGES * kStageBytes + 4 * kStripBytes) + wave * WN;
  if (s_first == col_range(cs, c_last)) {
    const float alpha = g_a * cs.gs[s_first];
    alpha_tab[lane] = alpha;
    alpha_tab[lane + 64] = alpha;
  } else {
    alpha_tab[lane] = col_alpha(g_a, cs, c_first + lane);
    alpha_tab[lane + 64] = col_alpha(g_a, cs, c_first + lane + 64);
  }
  // kGates (instantiated only for GEMMs that have gate columns): a wave
  // whose columns meet a gate range takes its own path and leaves; every
  // other wave takes the strip path below, the same code as without gates.
  // (A branch on the gate inside the unrolled strip loop made every wave of
  // a gated GEMM 18% slower.)  The gated path stages acc * alpha in fp32,
  // 16 rows x 64 columns at a time, in the wave's strip buffer, then applies
  // the gate functions in a rolled loop over it (one copy of their code) and
  // stores element by element.  No workgroup barrier follows, so leaving
  // early is safe.
  if constexpr (kGates) {
    static_assert(kStripBytes >= 16 * 64 * 4, "fp32 half strip");
    if (cols_gated(cs, c_first, c_last)) {
      float* fs = reinterpret_cast<float*>(smem + STAGES * kStageBytes + wave * kStripBytes);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int hc = 0; hc < 2; ++hc) {
            if ((r32 >> 4) == sub) {
#pragma unroll
              for (int j = 2 * hc; j < 2 * hc + 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                  const int cl = j * 32 + (v >> 2) * 8 + half * 4 + (v & 3);  // column within the wave's 128
                  fs[(r32 & 15) * 64 + cl - 64 * hc] = acc[j][i][v] * alpha_tab[cl];
                }
            }
            __asm__ volatile("" ::: "memory");  // other lanes' values are read below
            const int row0 = m0 + wave_m * WM + i * 32 + sub * 16, col0 = c_first + 64 * hc;
#pragma unroll 1
            for (int e = lane; e < 16 * 64; e += 64) {
              const int row = row0 + e / 64, col = col0 + e % 64;
              if (row < M && col < N) {
                const float o = col_gate(cs, col, fs[e]);
                if constexpr (kOutBf16)
                  reinterpret_cast<__bf16*>(y)[(int64_t)row * ldy + col] = (__bf16)o;
                else
                  reinterpret_cast<float*>(y)[(int64_t)row * ldy + col] = o;
              }
            }
            __asm__ volatile("" ::: "memory");  // reads done before the next pass writes
          }
      return;
    }
  }
  {
    uint8_t* strip = smem + STAGES * kStageBytes + wave * kStripBytes;
    constexpr int kChunksPerRow = kStripCols * kEsz / 16;
    constexpr int kChunkElems = 16 / kEsz;
    constexpr int kJPerPass = FN / kColPasses;
    // the lane's 64 column scales (4 per group of 4 columns), read once
    floatx4_t al[FN][4];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) al[j][g] = *reinterpret_cast<const floatx4_t*>(alpha_tab + j * 32 + g * 8 + half * 4);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int jp = 0; jp < kColPasses; ++jp) {  // columns [kStripCols jp, kStripCols (jp + 1)) of the wave
        uint8_t* rowp = strip + r32 * kStripRow;
#pragma unroll
        for (int jl = 0; jl < kJPerPass; ++jl)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int j = jp * kJPerPass + jl;
            const int col = jl * 32 + g * 8 + half * 4;  // within the strip
            if constexpr (kOutBf16) {
              typedef __bf16 bf4_t __attribute__((ext_vector_type(4)));
              bf4_t o;
#pragma unroll
              for (int t = 0; t < 4; ++t) o[t] = (__bf16)(acc[j][i][4 * g + t] * al[j][g][t]);
              *reinterpret_cast<bf4_t*>(rowp + col * kEsz) = o;
            } else {
              floatx4_t o;
#pragma unroll
              for (int t = 0; t < 4; ++t) o[t] = acc[j][i][4 * g + t] * al[j][g][t];
              *reinterpret_cast<floatx4_t*>(rowp + col * kEsz) = o;
            }
          }
        const int grow0 = m0 + wave_m * WM + i * 32;
        const int gcol0 = n0 + wave_n * WN + jp * kStripCols;
        constexpr int kQ = kStripRows * kChunksPerRow / 64;
        u32x4_t d[kQ];
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
          const int id = q * 64 + lane;
          d[q] = *reinterpret_cast<const u32x4_t*>(strip + (id / kChunksPerRow) * kStripRow + (id % kChunksPerRow) * 16);
        }
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
          const int id = q * 64 + lane;
          const int r = id / kChunksPerRow, c = id % kChunksPerRow;
          const int grow = grow0 + r, gcol = gcol0 + c * kChunkElems;
          if (grow < M) {
            out_t* dst = reinterpret_cast<out_t*>(y) + (int64_t)grow * ldy + gcol;
            if (vec_ok && gcol + kChunkElems <= N) {
              __builtin_nontemporal_store(d[q], reinterpret_cast<u32x4_t*>(dst));
            } else {
              const out_t* e = reinterpret_cast<const out_t*>(&d[q]);
              for (int t = 0; t < kChunkElems; ++t)
                if (gcol + t < N) dst[t] = e[t];
            }
          }
        }
        // Wait until the stores above have read their data registers
        // (expcnt) before the next strip's LDS reads may reuse them.  Without
        // it, when the compiler places the store data in AGPRs, a later
        // ds_read into the same AGPRs was seen to overwrite the data of a
        // store still in flight (wrong rows in the output).
        __builtin_amdgcn_s_waitcnt(0xCF0F);  // expcnt(0); vmcnt, lgkmcnt untouched
      }
    }
  }
}

// Decode kernel (M <= 64, K % 256 == 0): bound by the weight stream,
// N x K x 0.5625 bytes, which is read exactly once.
//
// A workgroup owns NB 16-row MFMA blocks of weight rows (the launcher picks
// NB = 1..4 so that the workgroups fill the 256 CUs with the fewest rounds:
// N = 12288 gives 256 workgroups of 48 rows) and all M rows of A; its
// kDecodeWaves (4) waves split K into contiguous parts of nt tiles of 256
// values.  Codes go straight into registers, D tiles ahead; only the scale
// bytes and the final reduction use LDS.
//
//  * One code load reads 8 rows x 128 contiguous bytes (lane L: row L % 8,
//    16-byte chunk L / 8), the pattern that reaches full HBM read bandwidth;
//    16 rows x 64 bytes per instruction loses about a quarter of it.
//  * v_mfma_f32_16x16x32_f16 wants lane L to hold row L % 16 of its 16-row
//    block.  Two loads X (rows 0-7) and Y (rows 8-15) are turned into that
//    layout with two DPP row shifts by 8 lanes: R0 = X in lanes 0-7 of every
//    16-lane row and Y shifted up in lanes 8-15 (chunk 2g for lane group g),
//    R1 = X shifted down in lanes 0-7 and Y in lanes 8-15 (chunk 2g + 1).
//    A is loaded and rearranged the same way (it stays in L2).
//  * The scale bytes of the wave's whole K range (16 bytes per row per tile)
//    are copied to LDS once, up front, in contiguous runs per row; read per
//    tile, they cost no extra memory requests.
//  * Rows >= M and rows >= N read zeros through the buffer bounds.
//  * kXIn = 1 (activations not yet quantized: bf16 values with the given
//    tensor scale, M <= kFusedRows, K <= kFusedMaxK): the ring also carries
//    activation values, one 16-value block per lane, and every 4 / Mp tiles
//    (Mp = M rounded up to a power of two) the wave quantizes the next 64
//    blocks of its K range into LDS (the same per-block arithmetic as the
//    quantize kernel, so the same bytes), and reads its A operand back in
//    MFMA layout.  That ALU work overlaps the weight loads in flight, which
//    bound the loop, and saves the separate quantize launch of a decode step.
//  * The waves' K-part partial sums are added through LDS in a fixed order
//    (deterministic), then scaled by RN32(g_a g_w) and stored.
// MB16 = number of 16-row blocks of A (1 to 4); NB = number of 16-row
// blocks of W; D = tiles in flight.
template <int MB16, int NB>
constexpr int decode_scale_rows() { return 16 * NB + 16 * MB16; }

// LDS bytes per wave and per K tile of its range: scale runs of W and A,
// plus the quantized A codes when the kernel quantizes A itself.
template <int MB16, int NB, int kXIn>
constexpr int decode_wave_bytes_per_tile() { return decode_scale_rows<MB16, NB>() * 16 + (kXIn ? 16 * MB16 * 128 : 0); }

template <int MB16, int NB, int D, int kXIn>
__global__ __launch_bounds__(64 * kDecodeWaves) void gemm_decode_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_gs,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, const ColScales cs,
    int M, int N, int K, void* __restrict__ y, int64_t ldy, bool out_bf16, int nt_max,
    const void* __restrict__ x, int64_t ldx) {
  constexpr int NW = 16 * NB;  // weight rows per workgroup
  constexpr int MA = 16 * MB16;
  constexpr int kTileBytes = 128, kTileScales = 16;  // per row, per 256-value tile
  constexpr int kLoads = 2 * NB + (kXIn ? 0 : 2 * MB16);  // code loads per tile
  static_assert(kXIn == 0 || (kXIn == 1 && MB16 == 1), "in-kernel quantization: bf16, M <= kFusedRows");
  static_assert(D * kLoads < 64, "vmcnt range");
  extern __shared__ __attribute__((aligned(16))) uint8_t dsmem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int q = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * NW;
  const uint32_t row_bytes = (uint32_t)K / 2, srow_bytes = (uint32_t)K / 16;
  const int kt = K / 256;
  const int t0 = (kt * wave) / kDecodeWaves, nt = (kt * (wave + 1)) / kDecodeWaves - t0;
  const int run = nt * kTileScales;  // scale bytes per row in this wave's range
  uint8_t* const wsl = dsmem + wave * decode_wave_bytes_per_tile<MB16, NB, kXIn>() * nt_max;  // [NW rows][run]
  uint8_t* const asl = wsl + NW * run;                                                    // [MA rows][run]
  uint8_t* const acl = asl + MA * run;  // kXIn: A codes [MA rows][nt * 128]

  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w_codes, (int64_t)N * row_bytes);
  const __amdgpu_buffer_rsrc_t rws = make_rsrc(w_scales, (int64_t)N * srow_bytes);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_codes, (int64_t)M * row_bytes);
  const __amdgpu_buffer_rsrc_t ras = make_rsrc(a_scales, (int64_t)M * srow_bytes);

  // Scale runs to LDS: 16-byte unit u = row * nt + t lands at u * 16, so one
  // instruction copies 64 consecutive units (whole row runs, contiguous).
  if (nt > 0) {
    const uint32_t inv = ((1u << 20) + nt - 1) / nt;  // u / nt == (u * inv) >> 20 for u * nt < 2^20
    for (int i = 0; i * 64 < NW * nt; ++i) {
      const uint32_t u = 64 * i + lane, row = (u * inv) >> 20, t = u - row * nt;
      if (u < (uint32_t)(NW * nt))
        lds_copy16(rws, (uint32_t)(n0 + row) * srow_bytes + (t0 + t) * kTileScales, 0, wsl + 64 * i * 16);
    }
    if constexpr (kXIn == 0) {
      for (int i = 0; i * 64 < MA * nt; ++i) {
        const uint32_t u = 64 * i + lane, row = (u * inv) >> 20, t = u - row * nt;
        if (u < (uint32_t)(MA * nt))
          lds_copy16(ras, row * srow_bytes + (t0 + t) * kTileScales, 0, asl + 64 * i * 16);
      }
    }
  }
  // kXIn: rows 0 .. Mp - 1 of A are quantized in the kernel, Mp = M rounded
  // up to 1, 2 or 4.  One pass of the wave quantizes 64 blocks of 16 values,
  // one per lane, covering P = 4 / Mp tiles: lane l takes block j = l % 16
  // of row r = (l / 16) % Mp of tile t + l / (16 Mp), for the tiles t with
  // t % P == 0.  The values travel in the ring with the weights of tile t;
  // the other tiles carry a dummy block (row 0, tile 0: always in bounds),
  // so the ring stays the same for every tile.  Rows M .. Mp - 1 are
  // quantized from that dummy block and stored as zeros; rows Mp .. 15 of
  // the A operand are cleared here, once.
  const int lmp = M == 1 ? 0 : (M == 2 ? 1 : 2), mp = 1 << lmp, pt = 4 >> lmp;
  const int xj = lane & 15, xr = (lane >> 4) & (mp - 1), xto = lane >> (4 + lmp);
  const uint16_t* const x_lane = reinterpret_cast<const uint16_t*>(x) + 16 * xj;
  if constexpr (kXIn != 0) {
    for (int o = 16 * lane; o < (MA - mp) * nt * kTileBytes; o += 64 * 16)
      *reinterpret_cast<u32x4_t*>(acl + mp * nt * kTileBytes + o) = u32x4_t{0, 0, 0, 0};
    for (int o = lane; o < (MA - mp) * run; o += 64) asl[mp * run + o] = 0;
  }

  // per-lane code offsets at tile 0 of this wave's K range
  uint32_t w_off[2 * NB], a_off[2 * MB16];
#pragma unroll
  for (int i = 0; i < 2 * NB; ++i)  // block i / 2, rows 8 (i % 2) .. + 7
    w_off[i] = (uint32_t)(n0 + 8 * i + (lane & 7)) * row_bytes + (uint32_t)(lane >> 3) * 16;
#pragma unroll
  for (int i = 0; i < 2 * MB16; ++i)
    a_off[i] = (uint32_t)(8 * i + (lane & 7)) * row_bytes + (uint32_t)(lane >> 3) * 16;

  struct Tile {
    u32x4_t x[kXIn ? 2 : 1];  // kXIn: the lane's 16 bf16 values
    u32x4_t w[2 * NB];
    u32x4_t a[2 * MB16];
  };
  // Tile t0 + t of this wave.  Tiles past the wave's range (t >= nt) are
  // read at an offset beyond every buffer's size: the loads return zeros
  // without touching memory, and the zero tile adds nothing to the sums.
  // That keeps the main loop branch-free, so the compiler can wait for each
  // tile individually instead of draining every load in flight.
  constexpr uint32_t kOutside = 0x80000000u;  // > any buffer size used here
  auto load = [&](Tile& T, int t) {
    const bool ok = t < nt;
    const uint32_t kc = (uint32_t)(t0 + t) * kTileBytes;
    if constexpr (kXIn != 0) {
      const int tq = t + xto;  // the lane's tile when t starts a pass
      const bool xok = (t & (pt - 1)) == 0 && tq < nt && xr < M;
      const u32x4_t* p = reinterpret_cast<const u32x4_t*>(
          xok ? x_lane + (int64_t)xr * ldx + (int64_t)(t0 + tq) * 256 : x_lane);
      T.x[0] = p[0];
      T.x[1] = p[1];
    }
#pragma unroll
    for (int i = 0; i < 2 * NB; ++i)
      T.w[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, ok ? w_off[i] + kc : kOutside, 0, 0);
    if constexpr (kXIn == 0) {
#pragma unroll
      for (int i = 0; i < 2 * MB16; ++i)
        T.a[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, ok ? a_off[i] + kc : kOutside, 0, 0);
    }
  };

  // kXIn: the tensor scale of A and an approximate 1 / (6 of it)
  const float gq = kXIn ? *a_gs : 1.0f;
  const float r6 = __builtin_amdgcn_rcpf(6.0f * gq);

  floatx4_t acc[NB][MB16];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int b = 0; b < MB16; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[j][b][v] = 0.0f;

  // X (rows 0-7) and Y (rows 8-15) of a 16-row block -> lane q holds row q:
  // r0 = chunk 2g, r1 = chunk 2g + 1 of the tile.
  auto to_mfma_rows = [](const u32x4_t& X, const u32x4_t& Y, u32x4_t& r0, u32x4_t& r1) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      r0[d] = (uint32_t)__builtin_amdgcn_update_dpp((int)X[d], (int)Y[d], 0x118, 0xF, 0xC, false);  // row_shr:8 -> lanes 8-15
      r1[d] = (uint32_t)__builtin_amdgcn_update_dpp((int)Y[d], (int)X[d], 0x108, 0xF, 0x3, false);  // row_shl:8 -> lanes 0-7
    }
  };

  // dequantized MFMA operands of the last three steps (see compute)
  half8_t wv[3][NB], av[3][MB16];
  auto compute = [&](const Tile& T, int t) {
    if constexpr (kXIn != 0) {
      // a pass: quantize the A blocks of tiles t .. t + P - 1 into LDS (codes
      // of block j of row r of tile u at r * 128 nt + 128 u + 8 j, scale at
      // r * run + 16 u + j); the same wave reads them back in MFMA layout
      if (t < nt && (t & (pt - 1)) == 0) {
        float v[16];
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[8 * k + 2 * e] = __uint_as_float(T.x[k][e] << 16);
            v[8 * k + 2 * e + 1] = __uint_as_float(T.x[k][e] & 0xFFFF0000u);
          }
        uint32_t w0, w1;
        uint32_t sc = quantize_block(v, gq, r6, w0, w1);
        if (xr >= M) w0 = w1 = sc = 0;
        const int tq = t + xto;
        if (tq < nt) {
          *reinterpret_cast<u32x2_t*>(acl + xr * (nt * kTileBytes) + tq * kTileBytes + 8 * xj) = u32x2_t{w0, w1};
          asl[xr * run + tq * kTileScales + xj] = (uint8_t)sc;
        }
      }
      // other lanes read these bytes below: keep every LDS read after the
      // writes (a wave's LDS accesses complete in issue order)
      __asm__ volatile("" ::: "memory");
    }
    // scale dword of the lane (4 blocks: chunks 2g and 2g + 1); phantom
    // tiles read the last real tile's scales (their codes are zero)
    const int ts = min(t, nt - 1) * kTileScales + 4 * g;
    uint32_t wsd[NB], asd[MB16];
#pragma unroll
    for (int j = 0; j < NB; ++j) wsd[j] = *reinterpret_cast<const uint32_t*>(wsl + (16 * j + q) * run + ts);
#pragma unroll
    for (int b = 0; b < MB16; ++b) asd[b] = *reinterpret_cast<const uint32_t*>(asl + (16 * b + q) * run + ts);
    u32x4_t wr[NB][2], ar[MB16][2];
#pragma unroll
    for (int j = 0; j < NB; ++j) to_mfma_rows(T.w[2 * j], T.w[2 * j + 1], wr[j][0], wr[j][1]);
    if constexpr (kXIn == 0) {
#pragma unroll
      for (int b = 0; b < MB16; ++b) to_mfma_rows(T.a[2 * b], T.a[2 * b + 1], ar[b][0], ar[b][1]);
    } else {
      // A already in LDS: row q, chunks 2g and 2g + 1 of the tile
      const int tc = min(t, nt - 1) * kTileBytes + 32 * g;
#pragma unroll
      for (int b = 0; b < MB16; ++b) {
        const uint8_t* p = acl + (16 * b + q) * (nt * kTileBytes) + tc;
        ar[b][0] = *reinterpret_cast<const u32x4_t*>(p);
        ar[b][1] = *reinterpret_cast<const u32x4_t*>(p + 16);
      }
    }
    // step s: chunk s / 4, dword s % 4; its scale is byte 2 (s / 4) + (s % 4) / 2
    // of the lane's scale dword.  Operands of step s + 1 are dequantized while
    // the MFMAs of step s issue, and the operands of step s - 1 are kept live
    // until the MFMAs of step s have issued (an empty asm that uses them).
    // An earlier version of this kernel produced wrong rows 8-15 of its
    // 16x16x32 MFMA blocks when a VALU wrote an MFMA's A/B registers right
    // behind its issue; the register allocator reuses those registers at once
    // unless they are still live, so the liveness is extended on purpose.
    // The last step's operands are kept live by the caller, past the next
    // refill.
    auto deq = [&](int s, int slot) {
      const int c = s >> 2, dw = s & 3, sb = 8 * (2 * c + (dw >> 1));
#pragma unroll
      for (int b = 0; b < MB16; ++b) av[slot][b] = dequant8(ar[b][c][dw], scale_pair((asd[b] >> sb) & 0xFFu));
#pragma unroll
      for (int j = 0; j < NB; ++j) wv[slot][j] = dequant8(wr[j][c][dw], scale_pair((wsd[j] >> sb) & 0xFFu));
    };
    deq(0, 0);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s + 1 < 8) deq(s + 1, (s + 1) % 3);
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int b = 0; b < MB16; ++b)
          acc[j][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv[s % 3][j], av[s % 3][b], acc[j][b], 0, 0, 0);
      if (s + 1 < 8) {
        constexpr int kMfma = NB * MB16, kValu = (8 * (NB + MB16) + kMfma - 1) / kMfma;
#pragma unroll
        for (int i = 0; i < kMfma; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);  // VALU
        }
      }
      // step s - 1's operands stay live until every instruction of step s
      // has issued (the barrier keeps the scheduler from moving MFMAs past
      // the asm)
      __builtin_amdgcn_sched_barrier(0);
      if (s > 0) keep_live(wv[(s + 2) % 3], av[(s + 2) % 3]);
    }
  };

  {
    Tile ring[D];
#pragma unroll
    for (int u = 0; u < D; ++u) {
      load(ring[u], u);
      __builtin_amdgcn_sched_barrier(0);  // issue the tiles in order
    }
    // The scale copies to LDS must have landed before the first scale read.
    // Waiting for every load in flight is the only count that holds however
    // the compiler orders the code loads around this point (a count of
    // D * kLoads is not: the compiler may issue part of the ring after the
    // wait, and the copies were then still in flight on a cold start).
    wait_vmcnt<0>();
    __asm__ volatile("" ::: "memory");  // no LDS read moves above the wait
    const int n_full = nt / D;
    for (int it = 0; it < n_full; ++it) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        compute(ring[u], it * D + u);
        // keep the refill right here: left alone, the scheduler sinks all
        // refills to the end of the loop body and every wait drains the queue
        __builtin_amdgcn_sched_barrier(0);
        load(ring[u], it * D + u + D);
        __builtin_amdgcn_sched_barrier(0);
        keep_live(wv[7 % 3], av[7 % 3]);  // last step's operands, past the refill
      }
    }
    // the last nt % D tiles are already in the ring
#pragma unroll
    for (int u = 0; u + 1 < D; ++u)
      if (u < nt - n_full * D) {
        compute(ring[u], n_full * D + u);
        __builtin_amdgcn_sched_barrier(0);
        keep_live(wv[7 % 3], av[7 % 3]);
      }
  }

  // Epilogue, compact on purpose: fully unrolled over every accumulator
  // block it was about 80 KB of straight-line code at MB16 = NB = 4, and
  // fetching it took longer than the main loop.  Every wave writes its K
  // part's sums to LDS (the scale area is free once all waves have passed
  // the barrier): part[w][m][c], m < MA rows of A, c < NW weight rows, the
  // 16-byte column quads of row m XOR-swizzled by m so that the 16 lanes of
  // one write or read phase hit distinct banks.  Then the 256 threads add
  // the four parts in a fixed order (deterministic), scale by RN32(g_a g_w)
  // and store 4 consecutive columns each, rows of NW columns contiguous.
  // The swizzle stays inside aligned groups of kSwz quads, kSwz the largest
  // power of two dividing the quads per row.
  constexpr int kQuads = NW / 4;                            // column quads per row
  constexpr int kSwz = kQuads & -kQuads;
  constexpr int kRowsPerPass = 64 * kDecodeWaves / kQuads;  // rows per pass of the 256 threads
  auto part_at = [&](int w, int m, int quad) -> floatx4_t* {
    return reinterpret_cast<floatx4_t*>(dsmem) + ((w * MA + m) * kQuads + (quad ^ (m & (kSwz - 1))));
  };
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int b = 0; b < MB16; ++b) *part_at(wave, 16 * b + q, 4 * j + g) = acc[j][b];
  __syncthreads();

  const int cq = tid % kQuads;
  const int n = n0 + 4 * cq;
  const float g_a = *a_gs;
  // one tensor scale for the workgroup's columns unless a column range ends
  // inside them
  const int s_first = col_range(cs, n0), s_last = col_range(cs, min(n0 + NW, N) - 1);
  float alpha[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) alpha[v] = s_first == s_last ? g_a * cs.gs[s_first] : col_alpha(g_a, cs, n + v);
  const bool gated = cols_gated(cs, n0, n0 + NW - 1);
  const bool vec_ok = (ldy % 4 == 0) && ((uintptr_t)y % 16 == 0) && n + 3 < N;
  const int m_end = min(MA, M);
#pragma unroll 1
  for (int m = tid < kRowsPerPass * kQuads ? tid / kQuads : m_end; m < m_end; m += kRowsPerPass) {
    floatx4_t t = *part_at(0, m, cq);
#pragma unroll
    for (int w = 1; w < kDecodeWaves; ++w) t += *part_at(w, m, cq);
    floatx4_t o;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      o[v] = t[v] * alpha[v];
      if (gated) o[v] = col_gate(cs, n + v, o[v]);
    }
    if (out_bf16) {
      __bf16* dst = reinterpret_cast<__bf16*>(y) + (int64_t)m * ldy + n;
      if (vec_ok) {
        typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
        bf16x4_t h;
#pragma unroll
        for (int v = 0; v < 4; ++v) h[v] = (__bf16)o[v];
        *reinterpret_cast<bf16x4_t*>(dst) = h;
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (n + v < N) dst[v] = (__bf16)o[v];
      }
    } else {
      float* dst = reinterpret_cast<float*>(y) + (int64_t)m * ldy + n;
      if (vec_ok) {
        *reinterpret_cast<floatx4_t*>(dst) = o;
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (n + v < N) dst[v] = o[v];
      }
    }
  }
}

// Dynamic LDS above 64 KiB has to be allowed per kernel before the launch.
bool allow_lds(const void* fn, size_t bytes) {
  if (bytes <= 64 * 1024) return true;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) == hipSuccess;
}

// LDS bytes of a decode launch: the per-wave scale runs, or the waves'
// partial sums if larger.
template <int MB16, int NB, int kXIn>
size_t decode_lds_bytes(int nt_max) {
  const size_t scales = (size_t)kDecodeWaves * decode_wave_bytes_per_tile<MB16, NB, kXIn>() * nt_max;
  const size_t red = (size_t)kDecodeWaves * (16 * NB) * (16 * MB16) * sizeof(float);
  return scales > red ? scales : red;
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_tiles(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
                        const uint8_t* w_codes, const uint8_t* w_scales, const ColScales& cs, int64_t M,
                        int64_t N, int64_t K, void* y, bool out_bf16, int64_t ldy, bool aligned,
                        hipStream_t stream) {
  constexpr int kThreads = (BM / WM) * (BN / WN) * 64;
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const dim3 grid((unsigned)tiles), block(kThreads);
  const int m = (int)M, n = (int)N, k = (int)K;
  if (aligned) {
    if (out_bf16)
      gemm_kernel<BM, BN, WM, WN, true, true><<<grid, block, 0, stream>>>(a_codes, a_scales, a_gs, w_codes, w_scales, cs, m, n, k, y, ldy);
    else
      gemm_kernel<BM, BN, WM, WN, true, false><<<grid, block, 0, stream>>>(a_codes, a_scales, a_gs, w_codes, w_scales, cs, m, n, k, y, ldy);
  } else {
    if (out_bf16)
      gemm_kernel<BM, BN, WM, WN, false, true><<<grid, block, 0, stream>>>(a_codes, a_scales, a_gs, w_codes, w_scales, cs, m, n, k, y, ldy);
    else
      gemm_kernel<BM, BN, WM, WN, false, false><<<grid, block, 0, stream>>>(a_codes, a_scales, a_gs, w_codes, w_scales, cs, m, n, k, y, ldy);
  }
  return hipGetLastError();
}

}  // namespace

namespace {

// Weight blocks of 16 rows per decode workgroup: the fewest rounds of 256
// workgroups times the blocks each one streams (ties: more blocks, so fewer
// workgroups re-read A).
int decode_blocks_per_wg(int64_t N) {
  const int64_t rb = (N + 15) / 16;
  int nb = 4;
  int64_t best = INT64_MAX;
  for (int c = 4; c >= 1; --c) {
    const int64_t cost = ((rb + c - 1) / c + 255) / 256 * c;
    if (cost < best) {
      best = cost;
      nb = c;
    }
  }
  return nb;
}

template <int MB, int kXIn>
size_t decode_lds_for(int nb, int nt_max) {
  switch (nb) {
    case 1: return decode_lds_bytes<MB, 1, kXIn>(nt_max);
    case 2: return decode_lds_bytes<MB, 2, kXIn>(nt_max);
    case 3: return decode_lds_bytes<MB, 3, kXIn>(nt_max);
    default: return decode_lds_bytes<MB, 4, kXIn>(nt_max);
  }
}

// Launches the decode kernel if the shape fits it (returns false otherwise).
// kXIn = 0: A is NVFP4 codes and scales; 1 / 2: A is bf16 / fp32 values
// quantized in the kernel (M <= 16).
template <int kXIn>
bool launch_decode(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs, const void* x, int64_t ldx,
                   const uint8_t* w_codes, const uint8_t* w_scales, const ColScales& cs, int64_t M, int64_t N,
                   int64_t K, void* y, bool out_bf16, int64_t ldy, hipStream_t stream, hipError_t* err) {
  const int nt_max = (int)((K / 256 + kDecodeWaves - 1) / kDecodeWaves);
  const int nb = decode_blocks_per_wg(N);
  const dim3 grid((unsigned)(((N + 15) / 16 + nb - 1) / nb)), block(64 * kDecodeWaves);
  const int m = (int)M, n = (int)N, k = (int)K;
#define NVFP4_DECODE_NB(MB, NBB, DD)                                                                              \
  do {                                                                                                             \
    const size_t lds = decode_lds_bytes<MB, NBB, kXIn>(nt_max);                                                    \
    if (lds > kDecodeMaxLds || !allow_lds((const void*)gemm_decode_kernel<MB, NBB, DD, kXIn>, lds)) return false; \
    gemm_decode_kernel<MB, NBB, DD, kXIn><<<grid, block, lds, stream>>>(                                           \
        a_codes, a_scales, a_gs, w_codes, w_scales, cs, m, n, k, y, ldy, out_bf16, nt_max, x, ldx);                \
    *err = hipGetLastError();                                                                                      \
    return true;                                                                                                   \
  } while (0)
#define NVFP4_DECODE(MB, DD)                        \
  do {                                              \
    switch (nb) {                                   \
      case 1: NVFP4_DECODE_NB(MB, 1, DD); break;    \
      case 2: NVFP4_DECODE_NB(MB, 2, DD); break;    \
      case 3: NVFP4_DECODE_NB(MB, 3, DD); break;    \
      default: NVFP4_DECODE_NB(MB, 4, DD); break;   \
    }                                               \
  } while (0)
  // Two tiles in flight per wave: with the compact epilogue, 2 measured
  // 7-10% faster than 3 at M <= 32 (fewer registers; N = 12288 / 12384,
  // K = 5120) and equal at M = 64, where 3 no longer fits in registers.
  if constexpr (kXIn != 0) {
    NVFP4_DECODE(1, 2);
  } else {
    if (M <= 16) NVFP4_DECODE(1, 2);
    else if (M <= 32) NVFP4_DECODE(2, 2);
    else if (M <= 48) NVFP4_DECODE(3, 2);  // rows past M still cost their dequantization
    else NVFP4_DECODE(4, 2);
  }
#undef NVFP4_DECODE
#undef NVFP4_DECODE_NB
  return false;
}

}  // namespace

hipError_t launch_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
                       const uint8_t* w_codes, const uint8_t* w_scales, const ColScales& cs,
                       int64_t M, int64_t N, int64_t K, void* y, bool out_bf16, int64_t ldy,
                       hipStream_t stream) {
  const bool aligned = (K % kBK == 0) && ((uintptr_t)a_codes % 16 == 0) && ((uintptr_t)w_codes % 16 == 0) &&
                       ((uintptr_t)a_scales % 8 == 0) && ((uintptr_t)w_scales % 8 == 0);
  const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
  const bool fits32 = M * (K / 2) < ((int64_t)1 << 31) && N * (K / 2) < ((int64_t)1 << 31);
  if (aligned && fits32 && big_tiles >= 256) {
    constexpr int kStages = 3;
    const dim3 grid((unsigned)big_tiles), block(256);
    const bool gates = cs.decay_hi > cs.decay_lo || cs.write_hi > cs.write_lo;
#define NVFP4_STREAM(BF16, GATES)                                                                           \
  gemm_stream_kernel<kStages, BF16, GATES, false><<<grid, block, 0, stream>>>(a_codes, a_scales, a_gs, w_codes, \
                                                                              w_scales, cs, (int)M, (int)N,  \
                                                                              (int)K, y, ldy, SwigluOut{})
    if (out_bf16) {
      if (gates) NVFP4_STREAM(true, true);
      else NVFP4_STREAM(true, false);
    } else {
      if (gates) NVFP4_STREAM(false, true);
      else NVFP4_STREAM(false, false);
    }
#undef NVFP4_STREAM
    return hipGetLastError();
  }
  // decode: buffer offsets of rows up to N + 63 must stay below 2^31, and
  // the scale runs of the longest K part must fit in LDS
  const bool fits_decode = (N + 64) * (K / 2) < ((int64_t)1 << 31) && M * (K / 2) < ((int64_t)1 << 31);
  if (aligned && fits_decode && M <= 64 && K % 256 == 0) {
    hipError_t err = hipSuccess;
    if (launch_decode<0>(a_codes, a_scales, a_gs, nullptr, 0, w_codes, w_scales, cs, M, N, K, y, out_bf16, ldy,
                         stream, &err))
      return err;
  }
  return launch_tiles<128, 128, 64, 64>(a_codes, a_scales, a_gs, w_codes, w_scales, cs, M, N, K, y,
                                        out_bf16, ldy, aligned, stream);
}

hipError_t launch_gemm_swiglu_quantize(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
                                       const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gs,
                                       int64_t M, int64_t F, int64_t K, const SwigluOut& out, hipStream_t stream) {
  ColScales cs{};
  cs.gs = w_gs;
  cs.n = 1;
  cs.end[0] = (int)(2 * F);
  const int64_t tiles = ((M + 255) / 256) * ((2 * F + 255) / 256);
  gemm_stream_kernel<3, false, false, true><<<dim3((unsigned)tiles), dim3(256), 0, stream>>>(
      a_codes, a_scales, a_gs, w_codes, w_scales, cs, (int)M, (int)(2 * F), (int)K, nullptr, 0, out);
  return hipGetLastError();
}

bool quantize_gemm_fused_fits(int64_t M, int64_t N, int64_t K, bool in_bf16) {
  if (!in_bf16 || M < 1 || M > kFusedRows || K % 256 != 0) return false;
  if (K > kFusedMaxK) return false;
  if ((N + 64) * (K / 2) >= ((int64_t)1 << 31)) return false;
  return decode_lds_for<1, 1>(decode_blocks_per_wg(N), (int)((K / 256 + kDecodeWaves - 1) / kDecodeWaves)) <=
         kDecodeMaxLds;
}

hipError_t launch_quantize_gemm_fused(const void* x, bool in_bf16, int64_t ldx, const float* a_gs,
                                      const uint8_t* w_codes, const uint8_t* w_scales, const ColScales& cs,
                                      int64_t M, int64_t N, int64_t K, void* y, bool out_bf16, int64_t ldy,
                                      hipStream_t stream) {
  hipError_t err = hipErrorInvalidValue;
  if (!in_bf16) return hipErrorInvalidValue;
  const bool ok = launch_decode<1>(nullptr, nullptr, a_gs, x, ldx, w_codes, w_scales, cs, M, N, K, y, out_bf16,
                                   ldy, stream, &err);
  return ok ? err : hipErrorInvalidConfiguration;
}

}  // namespace nvfp4
