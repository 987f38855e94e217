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
//  * Packed codes and scale bytes are staged through LDS or registers (4.5
//    bits per value, a quarter of the bytes an fp16 tile would need) and
//    every wave dequantizes its own operand fragments in registers: per 8
//    values one hardware FP4->fp16 conversion per byte and one packed fp16
//    multiply per pair by the block scale.  The streaming and decode kernels
//    convert two E4M3 scale bytes at a time to exact fp16 values with the
//    hardware fp8 conversion and let the multiply's operand select pick the
//    half; the generic kernel takes the scale as fp16 bits (scale byte << 7
//    = E4M3 value * 2^-8, codes converted with scale 2^8).  All exact.
//  * Within an MFMA the K order is free as long as A and W agree, and the 8
//    values a lane supplies to one MFMA always sit inside one 16-value block,
//    i.e. one scale.  The large shapes run on v_mfma_f32_16x16x32_f16, decode
//    on the same instruction, the generic fallback on v_mfma_f32_32x32x16_f16.
//  * The RN32(g_a g_w) multiply and the fp32 or bf16 (RNE) conversion happen
//    in the epilogue, straight from the accumulators.
#include <algorithm>
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

// 8 consecutive codes -> 8 exact fp16 values, multiplied by half `h` of the
// fp16 scale pair sp (the multiply's operand select picks the half, so the
// pair costs no extraction).
__device__ __forceinline__ half8_t dequant8_sel(uint32_t codes, half2_t sp, int h) {
  const half2_t sc = h ? __builtin_shufflevector(sp, sp, 1, 1) : __builtin_shufflevector(sp, sp, 0, 0);
  const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * sc;
  const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * sc;
  const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * sc;
  const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * sc;
  half8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Marks MFMA operands as still in use at this point of the program, so the
// register allocator cannot hand their registers to a new value before it.
//
// Why: a VALU instruction that writes an MFMA's A/B source registers right
// behind the MFMA's issue was seen to corrupt the MFMA's operand on gfx950
// (rows 8-15 of a v_mfma_f32_16x16x32_f16 A operand), and the compiler
// inserts no wait states for that pattern (its hazard model covers only
// the C operand).  Every kernel here therefore keeps each step's operands
// live until the next step's MFMAs have issued, and ends its MFMA work with
// mfma_drain(); a CPU test scans the compiled gfx950 code of every kernel
// and requires at least 4 instructions between an MFMA and any VALU write
// to its A/B registers.
template <int A, int B>
__device__ __forceinline__ void keep_live(const half8_t (&x)[A], const half8_t (&y)[B]) {
#pragma unroll
  for (int i = 0; i < A; ++i) __asm__ volatile("" ::"v"(x[i]));
#pragma unroll
  for (int i = 0; i < B; ++i) __asm__ volatile("" ::"v"(y[i]));
}

// After a kernel's last MFMA: 8 wait states, so that no epilogue VALU can
// write a register the last MFMAs read right behind their issue.
__device__ __forceinline__ void mfma_drain() {
  __builtin_amdgcn_sched_barrier(0);
  __asm__ volatile("s_nop 7");
  __builtin_amdgcn_sched_barrier(0);
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
    // Three operand slots: step kk reads slot kk % 3 and writes kk + 1's
    // operands into the slot step kk - 2 read, while step kk - 1's operands
    // are kept live (keep_live) until step kk's MFMAs have issued, so no
    // VALU result lands in a register an MFMA read a few instructions before
    // (see keep_live).
    half8_t af[3][FM], wf[3][FN];
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
      const int cur = kk % 3;
      if (kk + 1 < 8) dequant_step(kk + 1, (kk + 1) % 3);
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
      __builtin_amdgcn_sched_barrier(0);
      if (kk > 0) keep_live(af[(kk + 2) % 3], wf[(kk + 2) % 3]);
    }
    // the last step's operands stay live past the refill's LDS stores
    __builtin_amdgcn_sched_barrier(0);
    keep_live(af[7 % 3], wf[7 % 3]);
    mfma_drain();

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

// v_mfma_f32_16x16x32_f16 with the accumulator pinned in AGPRs (dst = srcC).
// Written as inline asm because the compiler, given 64 such accumulators
// through the builtin, shuttled them between AGPRs and VGPRs on every pass
// of the loop (256 copies each way per 256 matrix instructions).  The
// compiler does not track hazards into inline asm, so the kernel keeps its
// own distances: no accumulator is read by the next 63 matrix instructions,
// every operand is written at least 8 matrix instructions before its reader
// and at least 8 after its last reader, the accumulators are zeroed long
// before the first one, and mfma16_drain() runs before any other use.
__device__ __forceinline__ void mfma16(floatx4_t& acc, const half8_t& a, const half8_t& b) {
  __asm__ volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// 24 wait states after the last matrix instruction, before its results (or
// its operand registers) are touched by anything else.
__device__ __forceinline__ void mfma16_drain() {
  __builtin_amdgcn_sched_barrier(0);
  __asm__ volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
  __builtin_amdgcn_sched_barrier(0);
}

// Streaming kernel for the large shapes (K % 128 == 0, aligned operands) on
// 16x16x32 matrix instructions: the plain epilogue (every output column
// times its range's RN32(g_a g_w)), with kGates the GDN gate functions on
// the gate columns, with kSplit the K parts of a split tail, and with
// kSwiglu the MLP's gate/up projection: h = silu(gate) up, quantized to
// NVFP4 for the down projection in the epilogue (W = [gate; up], 128 output
// columns per tile).
//
//  * 256 x 256 output tile per workgroup, 4 waves of 128 x 128 (8 x 8 blocks
//    of 16 x 16), accumulators in AGPRs; tile order as tile_coords().
//  * K steps of 128 values stream through a 3-deep LDS ring filled by direct
//    global -> LDS copies (no VGPR staging), 3 K steps ahead; 16-byte code
//    chunks of each row XOR-swizzled by chunk_swizzle(row).
//
// Why 16x16x32: with operands of dequantized NVFP4 values that change every
// instruction, all CUs busy and the dequantization's VALU work interleaved
// at this kernel's ratio, v_mfma_f32_16x16x32_f16 sustained 1,990 TFLOP/s on
// an MI355X against 1,619 for v_mfma_f32_32x32x16_f16 (register-only probe,
// same box, back to back): the board holds its power limit under this load,
// and the 16x16 form moves fewer accumulator bytes per multiply-add.
//
//  * Operand layout: lane (r16 = L % 16, q = L / 16) supplies 8 K values of
//    row r16 of a 16-row block, for W (the instruction's A operand) and A
//    alike; its accumulators hold output columns 4q .. 4q + 3 of the W block
//    for output row r16 of the A block.
//  * K mapping: a stage of 128 K values is used in 4 steps of 32.  Lane
//    group q owns the 32 values of 16-byte chunk q of each row (scale blocks
//    2q, 2q + 1) and reads them 8 bytes at a time: pair u (steps 2u, 2u + 1)
//    is the chunk's half h = (u + q) & 1, so the 64 lanes of one 8-byte read
//    hit distinct LDS banks (rows 4 apart share banks; the chunk swizzle
//    separates them, the rotation by q the lane groups).  At step t a lane
//    uses dword t & 1 of its pair, the same K values for both operands.
//  * Registers: pair 0 and pair 1 of the codes (64 VGPRs); A operands
//    double-buffered by step (64), dequantized one step ahead; W operands in
//    4 rotating buffers, block j + 1 dequantized during block j's MFMAs.  A
//    VALU write into an operand register therefore comes at least 12 MFMAs
//    after the register's last MFMA read.
//  * Per stage: the next stage's pair 0 and scale bytes are read after the
//    mid-tile barrier (step 2), pair 1 of the current stage during step 0.
template <int STAGES, bool kOutBf16, bool kGates, bool kSplit, bool kSwiglu = false>
__global__ __launch_bounds__(256) void gemm_stream16_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_gs,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, const ColScales cs,
    int M, int N, int K, void* __restrict__ y, int64_t ldy, const SplitTail sp, const SwigluOut sw) {
  constexpr int BM = 256, BN = 256, WM = 128, WN = 128, FB = 8;  // 16-row blocks per operand per wave
  constexpr int kCodeBytes = BM * kRowBytes;          // 16 KiB per operand per stage
  constexpr int kStageScaleBytes = BM * kScaleBytes;  // 2 KiB per operand per stage
  constexpr int kStageBytes = 2 * kCodeBytes + 2 * kStageScaleBytes;
  constexpr int kLoadsPerStage = 12;
  using out_t = typename std::conditional<kOutBf16, __bf16, float>::type;
  constexpr int kEsz = sizeof(out_t);
  constexpr int kStripRows = 32;
  constexpr int kColPasses = kOutBf16 ? 1 : 2;
  constexpr int kStripCols = WN / kColPasses;
  constexpr int kStripRow = kStripCols * kEsz + 16;
  constexpr int kStripBytes = kStripRows * kStripRow;
  static_assert(STAGES >= 3, "ring depth");
  static_assert((STAGES - 1) * kLoadsPerStage < 64, "vmcnt range");
  // Ring layout: the A codes of all stages, then the W codes, the A scales
  // and the W scales, so that every LDS read below is a per-lane base
  // register plus an immediate offset under 64 KiB.
  constexpr int kACode = 0, kWCode = STAGES * kCodeBytes, kAScale = 2 * STAGES * kCodeBytes,
                kWScale = kAScale + STAGES * kStageScaleBytes;
  static_assert(kWScale + STAGES * kStageScaleBytes == STAGES * kStageBytes, "ring size");
  static_assert((STAGES - 1) * kCodeBytes + 16 * kRowBytes * 8 < 65536, "code read offsets fit the immediate");
  constexpr int kAlphaBytes = WN * 4;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * kStageBytes + 4 * kStripBytes + 4 * kAlphaBytes];
  uint8_t* const ring = smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_m = wave >> 1, wave_n = wave & 1;
  const int r16 = lane & 15, q = lane >> 4;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int64_t row_bytes = K / 2, srow_bytes = K / 16;
  const int ksteps = K / kBK;
  const bool vec_ok = ((uintptr_t)y % 16 == 0) && ((ldy * kEsz) % 16 == 0);

  // Copies: wave w copies rows 64w .. 64w + 63 of both operands (codes with
  // 4 instructions of 16 rows x 4 swizzled 16-byte chunks, scales with 2 of
  // 32 rows x 2 dwords); rows past an operand are clamped to its last row.
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_codes, (int64_t)M * row_bytes);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w_codes, (int64_t)N * row_bytes);
  const __amdgpu_buffer_rsrc_t ras = make_rsrc(a_scales, (int64_t)M * srow_bytes);
  const __amdgpu_buffer_rsrc_t rws = make_rsrc(w_scales, (int64_t)N * srow_bytes);
  uint32_t a_off[4], w_off[4], as_off[2], ws_off[2];
  // W row of tile row r (0 .. 255).  Plain: row n0 + r, clamped to the last
  // row.  kSwiglu (W = [gate (F rows); up (F rows)], N = 2F): the tile's rows
  // are the gate and up rows of its 128 output columns c0 = n0 / 2 .. + 127,
  // in 16-row blocks: tile row r is in wave half wn = r / 128 and that
  // wave's W block j = (r / 16) % 8, for output column c0 + 64 wn + 16 (j / 2)
  // + r % 16, a gate row for even j and an up row for odd j.  So a lane's
  // accumulator blocks 2p (gate) and 2p + 1 (up) hold the same output
  // elements.  Columns past F repeat column F - 1 (never stored).
  auto w_row = [&](int n0, int r) -> int {
    if constexpr (kSwiglu) {
      const int col = n0 / 2 + 64 * (r >> 7) + 16 * ((r >> 5) & 3) + (r & 15);
      return min(col, sw.F - 1) + (((r >> 4) & 1) ? sw.F : 0);
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
  auto issue_one = [&](int ks, int slot, int g) {
    const uint32_t kc = (uint32_t)ks * kRowBytes, kscl = (uint32_t)ks * kScaleBytes;
    uint8_t* const codes = ring + slot * kCodeBytes;
    uint8_t* const scales = ring + slot * kStageScaleBytes;
    if (g < 4) lds_copy16(ra, a_off[g], kc, codes + kACode + (wave * 64 + 16 * g) * kRowBytes);
    else if (g < 8) lds_copy16(rw, w_off[g - 4], kc, codes + kWCode + (wave * 64 + 16 * (g - 4)) * kRowBytes);
    else if (g < 10) lds_copy4(ras, as_off[g - 8], kscl, scales + kAScale + (wave * 64 + 32 * (g - 8)) * kScaleBytes);
    else lds_copy4(rws, ws_off[g - 10], kscl, scales + kWScale + (wave * 64 + 32 * (g - 10)) * kScaleBytes);
  };

  // Accumulators, zeroed in AGPRs long before the first matrix instruction
  // reads them (the instructions are inline asm, which the compiler's hazard
  // tracking does not see into).
  floatx4_t acc[FB][FB];  // acc[j][i]: W block j (output columns) x A block i (output rows)
#pragma unroll
  for (int j = 0; j < FB; ++j)
#pragma unroll
    for (int i = 0; i < FB; ++i) {
      acc[j][i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
      __asm__ volatile("" : "+a"(acc[j][i]));
    }

  // Workgroup -> tile, and the tile's K steps [k_first, k_first + k_count):
  // all of them, or (kSplit) part `unit % splits` of tail tile `unit / splits`.
  int bid = blockIdx.x, k_first = 0, k_count = ksteps;
  if constexpr (kSplit) {
    const int unit = blockIdx.x, piece = unit % sp.splits;
    bid = sp.full + unit / sp.splits;
    k_first = ksteps * piece / sp.splits;
    k_count = ksteps * (piece + 1) / sp.splits - k_first;
  }
  int tile_m, tile_n;
  tile_coords(bid, tiles_m, tiles_n, tile_m, tile_n);
  const int m0 = tile_m * BM, n0 = tile_n * BN;
  set_sources(m0, n0);
  // The ring always holds STAGES copies in flight or landed; past the last
  // K step the copies repeat it into a slot nobody reads again.
#pragma unroll
  for (int s = 0; s < STAGES; ++s)
#pragma unroll
    for (int g = 0; g < kLoadsPerStage; ++g) issue_one(k_first + min(s, k_count - 1), s, g);

  // Per-lane LDS offsets within a stage.  Row R = 128 w + 16 b + r16 of an
  // operand: chunk q sits at chunk position q ^ chunk_swizzle(R), and
  // chunk_swizzle(R) = chunk_swizzle(r16) ^ 2 (b & 1).
  const int s0 = chunk_swizzle(r16);
  uint32_t lo[2][2];  // [block parity][pair]
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int u = 0; u < 2; ++u) lo[p][u] = r16 * kRowBytes + 16 * (q ^ s0 ^ (2 * p)) + 8 * ((u + q) & 1);
  const uint32_t lsc = r16 * kScaleBytes + 2 * q;  // the lane's scale bytes 2q, 2q + 1 of its row
  // The lane's LDS bases, opaque to the compiler so that it keeps them in
  // registers instead of adding large stage offsets before every read.
  uint32_t abase[2][2], wbase[2][2];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      abase[p][u] = kACode + wave_m * WM * kRowBytes + lo[p][u];
      wbase[p][u] = kWCode + wave_n * WN * kRowBytes + lo[p][u];
      __asm__ volatile("" : "+v"(abase[p][u]), "+v"(wbase[p][u]));
    }
  uint32_t asbase = kAScale + wave_m * WM * kScaleBytes + lsc, wsbase = kWScale + wave_n * WN * kScaleBytes + lsc;
  __asm__ volatile("" : "+v"(asbase), "+v"(wsbase));
  // v_perm selector packing the scale bytes of blocks 2k, 2k + 1 into one
  // dword, swapped for odd q so that pair u's byte is byte u (block 2k) and
  // byte 2 + u (block 2k + 1)
  const uint32_t psel = (q & 1) ? 0x04050001u : 0x05040100u;

  u32x2_t ra2[2][FB], rw2[2][FB];  // code pairs u = 0, 1 of the lane's rows
  uint32_t xs[2 * FB];
  // block scales as exact fp16 values: asp[slot][b] = (scale of block b at
  // pair 0, at pair 1) of the lane's rows in ring slot `slot` (one set per
  // slot, so the unrolled stage loop rotates no registers)
  half2_t asp[STAGES][FB], wsp[STAGES][FB];
  half8_t af[2][FB], wf[4];
  half2_t ta[4], tw[4];

  auto read_pair = [&](int slot, int u, int g) {  // g < 8: A block g, else W block g - 8
    const int b = g & 7;
    const uint32_t off = slot * kCodeBytes + 16 * kRowBytes * b;
    if (g < FB)
      ra2[u][b] = *reinterpret_cast<const u32x2_t*>(ring + abase[b & 1][u] + off);
    else
      rw2[u][b] = *reinterpret_cast<const u32x2_t*>(ring + wbase[b & 1][u] + off);
  };
  auto read_scale = [&](int slot, int g) {
    const int b = g & 7;
    xs[g] = *reinterpret_cast<const uint16_t*>(ring + (g < FB ? asbase : wsbase) + slot * kStageScaleBytes +
                                               16 * kScaleBytes * b);
  };
  // k = 0..7: the scale bytes of 16-row blocks 2k', 2k' + 1 (k' = k % 4) of A
  // (k < 4) or W packed into one dword, then converted to two fp16 pairs
  auto pack_scales = [&](half2_t (&ap)[FB], half2_t (&wp)[FB], int k) {
    const int kk = k & 3;
    const uint32_t d = k < 4 ? __builtin_amdgcn_perm(xs[2 * kk + 1], xs[2 * kk], psel)
                             : __builtin_amdgcn_perm(xs[2 * kk + 9], xs[2 * kk + 8], psel);
    const half2_t lo2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d, 1.0f, false);
    const half2_t hi2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d, 1.0f, true);
    if (k < 4) {
      ap[2 * kk] = lo2;
      ap[2 * kk + 1] = hi2;
    } else {
      wp[2 * kk] = lo2;
      wp[2 * kk + 1] = hi2;
    }
  };
  auto cvt = [&](uint32_t codes, int k) -> half2_t {
    if (k == 0) return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0);
    if (k == 1) return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1);
    if (k == 2) return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2);
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3);
  };
  // piece k (0..7) of dequantizing 8 codes into dst: 4 conversions, then 4
  // multiplies by half u of the block's scale pair sp (selected by the
  // multiply's operand select, no extra instruction)
  auto piece = [&](half2_t (&tmp)[4], uint32_t codes, half2_t sp, int u, half8_t& dst, int k) {
    if (k < 4) {
      tmp[k] = cvt(codes, k);
    } else {
      const half2_t s = u ? __builtin_shufflevector(sp, sp, 1, 1) : __builtin_shufflevector(sp, sp, 0, 0);
      const half2_t v = tmp[k - 4] * s;
      dst[2 * (k - 4)] = v[0];
      dst[2 * (k - 4) + 1] = v[1];
    }
  };

  // first K step: wait for its copies, read its pair 0 and scales, and
  // dequantize step 0 of A and block 0 of W
  wait_vmcnt<(STAGES - 1) * kLoadsPerStage>();
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int g = 0; g < 2 * FB; ++g) read_pair(0, 0, g);
#pragma unroll
  for (int g = 0; g < 2 * FB; ++g) read_scale(0, g);
#pragma unroll
  for (int k = 0; k < 8; ++k) pack_scales(asp[0], wsp[0], k);
#pragma unroll
  for (int b = 0; b < FB; ++b)
#pragma unroll
    for (int k = 0; k < 8; ++k) piece(ta, ra2[0][b][0], asp[0][b], 0, af[0][b], k);
#pragma unroll
  for (int k = 0; k < 8; ++k) piece(tw, rw2[0][0][0], wsp[0][0], 0, wf[0], k);
  // block 1: converted here, multiplied in the first slots of the loop
#pragma unroll
  for (int k = 0; k < 4; ++k) piece(tw, rw2[0][1][0], wsp[0][1], 0, wf[1], k);
  // the first operands are in their registers, and 8 wait states pass,
  // before the first matrix instruction
  keep_live(af[0], wf);
  __asm__ volatile("s_nop 7");
  __builtin_amdgcn_sched_barrier(0);

  // One K step of 128 values in ring slot `slot` (a compile-time constant,
  // so every LDS address is a loop-invariant register plus an immediate).
  auto run_stage = [&](int it, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value, next_slot = (slot + 1) % STAGES;
    const int refill = k_first + min(it + STAGES, k_count - 1);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t == 1 || t == 3) {
        // the LDS reads issued a step earlier (pair 1 in step 0; the next
        // stage's scales and pair 0 in step 2) have long returned: one wait
        // here instead of one in front of each first use
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt untouched
        __builtin_amdgcn_sched_barrier(0);
      }
      if (t == 2) {
        // mid-stage: the next stage has landed (own copies + barrier) and
        // every wave has read this slot (pair 1 in step 0), so the slot is
        // refilled; a bare s_barrier keeps the other copies in flight
        wait_vmcnt<(STAGES - 2) * kLoadsPerStage>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int n = 0; n < FB * FB; ++n) {
        const int j = n >> 3, i = n & 7;
        mfma16(acc[j][i], wf[j & 3], af[t & 1][i]);
        // A block j of the next step (the next stage's step 0 at t == 3)
        if (t < 3)
          piece(ta, ra2[(t + 1) >> 1][j][(t + 1) & 1], asp[slot][j], (t + 1) >> 1, af[(t + 1) & 1][j], i);
        else
          piece(ta, ra2[0][j][0], asp[next_slot][j], 0, af[0][j], i);
        // W, 4 slots behind A so that no slot holds both scale extractions:
        // slots 4-7 of block j convert block j + 2, slots 0-3 multiply block
        // j + 1 (converted in block j - 1); blocks past 7 are the next
        // step's (the next stage's at t == 3)
        {
          const int jb = i < 4 ? j + 1 : j + 2, kw = i < 4 ? i + 4 : i - 4;
          if (jb < 8)
            piece(tw, rw2[t >> 1][jb][t & 1], wsp[slot][jb], t >> 1, wf[jb & 3], kw);
          else if (t < 3)
            piece(tw, rw2[(t + 1) >> 1][jb - 8][(t + 1) & 1], wsp[slot][jb - 8], (t + 1) >> 1, wf[jb & 3], kw);
          else
            piece(tw, rw2[0][jb - 8][0], wsp[next_slot][jb - 8], 0, wf[jb & 3], kw);
        }
        if (t == 0 && n < 2 * FB) read_pair(slot, 1, n);  // pair 1 of this stage
        if (t == 2 && n < kLoadsPerStage) issue_one(refill, slot, n);
        if (t == 2 && n >= 12 && n < 12 + 2 * FB) read_scale(next_slot, n - 12);    // the next stage's scales
        if (t == 2 && n >= 28 && n < 28 + 2 * FB) read_pair(next_slot, 0, n - 28);  // and its pair 0
        if (t == 2 && n >= 48 && (n & 1) == 0) pack_scales(asp[next_slot], wsp[next_slot], (n - 48) >> 1);
        // the operands of the matrix instruction 4 slots back stay allocated
        // until here, so no new value lands in their registers right behind
        // their last read (the previous step's at n < 4)
        if (n >= 4) {
          __asm__ volatile("" ::"v"(wf[((n - 4) >> 3) & 3]), "v"(af[t & 1][(n - 4) & 7]));
        } else {
          __asm__ volatile("" ::"v"(wf[3]), "v"(af[(t + 1) & 1][4 + n]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // The next stage's first operands (and W block 1's conversions), its
    // code pair 0 and its scale pairs are complete here, ahead of the loop's
    // exit test: otherwise the compiler sinks the work that only the next
    // stage uses past the test.  Sunk multiplies landed right in front of
    // the matrix instructions that read them, with no wait states between;
    // sunk LDS reads and scale conversions bunch up at the next stage's
    // start instead of running in their slots.
    keep_live(af[0], wf);
    __asm__ volatile("" ::"v"(tw[0]), "v"(tw[1]), "v"(tw[2]), "v"(tw[3]));
#pragma unroll
    for (int b = 0; b < FB; ++b)
      __asm__ volatile("" ::"v"(ra2[0][b]), "v"(rw2[0][b]), "v"(asp[next_slot][b]), "v"(wsp[next_slot][b]));
    __builtin_amdgcn_sched_barrier(0);
  };
  static_assert(STAGES == 3, "the stage loop is unrolled by the ring depth");
  // k_count >= 1; a pass that runs out of K steps leaves the loop at once,
  // so the loop's back edge comes only from a full pass of STAGES steps
  for (int it = 0;; it += STAGES) {
    run_stage(it, std::integral_constant<int, 0>{});
    if (it + 1 >= k_count) break;
    run_stage(it + 1, std::integral_constant<int, 1>{});
    if (it + 2 >= k_count) break;
    run_stage(it + 2, std::integral_constant<int, 2>{});
    if (it + 3 >= k_count) break;
  }
  mfma16_drain();
  wait_vmcnt<0>();  // the repeated copies past the last K step

  if constexpr (kSplit) {
    // one K part of a split tile: its raw fp32 sums, row-major [256 x 256],
    // for the adding kernel; no LDS is touched, so no barrier
    float* dst = sp.part + (size_t)blockIdx.x * (256 * 256);
#pragma unroll
    for (int j = 0; j < FB; ++j)
#pragma unroll
      for (int i = 0; i < FB; ++i) {
        const int row = wave_m * WM + 16 * i + r16, col = wave_n * WN + 16 * j + 4 * q;
        *reinterpret_cast<floatx4_t*>(dst + row * 256 + col) = acc[j][i];
      }
    return;
  }
  __syncthreads();  // every wave is done with the ring

  if constexpr (kSwiglu) {
    // h = silu(g) u of the wave's 64 output columns c_out .. + 63 (g, u =
    // acc RN32(g_a g_w) of W blocks 2p and 2p + 1), staged in fp32 in the
    // wave's strip buffer 32 rows at a time (rows of 64 values padded to 68,
    // so that the 16 rows of one write phase spread over the banks): 128
    // blocks of 16 values, two per lane.  Each lane then quantizes its
    // blocks with the quantize kernel's arithmetic and stores 8 code bytes
    // and 1 scale byte per block (and, if asked, the 16 fp32 values).
    constexpr int kHRow = 68;  // floats per staged row
    static_assert(kStripBytes >= 32 * kHRow * 4, "fp32 strip of 32 x 64 (padded)");
    const float alpha = *a_gs * cs.gs[0];
    const int c_out = n0 / 2 + 64 * wave_n;
    float* const fs = reinterpret_cast<float*>(smem + STAGES * kStageBytes + wave * kStripBytes);
    const float hg = *sw.gs, r6 = __builtin_amdgcn_rcpf(6.0f * hg);
    const int qr = lane >> 2, qb = lane & 3;  // the lane's blocks: rows qr and 16 + qr, 16-column block qb
    if (c_out < sw.F) {
#pragma unroll
      for (int s = 0; s < FB / 2; ++s) {
        // rows of A blocks 2s, 2s + 1: every lane writes its values
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
          for (int pp = 0; pp < FB / 2; ++pp) {
            floatx4_t h4;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              h4[e] = silu_fast(acc[2 * pp][2 * s + ii][e] * alpha) * (acc[2 * pp + 1][2 * s + ii][e] * alpha);
            *reinterpret_cast<floatx4_t*>(fs + (16 * ii + r16) * kHRow + 16 * pp + 4 * q) = h4;
          }
        __asm__ volatile("" ::: "memory");  // other lanes' values are read below
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          const int row = m0 + wave_m * WM + 32 * s + 16 * sub + qr;
          const floatx4_t* src = reinterpret_cast<const floatx4_t*>(fs + (16 * sub + qr) * kHRow + 16 * qb);
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
              for (int e = 0; e < 4; ++e)
                dst[e] = floatx4_t{vals[4 * e], vals[4 * e + 1], vals[4 * e + 2], vals[4 * e + 3]};
            }
          }
        }
        // the stores above must have read their data registers before the
        // next pass's LDS reads may land in them (a later ds_read into the
        // registers of a store still in flight was seen to overwrite its data)
        __builtin_amdgcn_s_waitcnt(0xCF0F);  // expcnt(0); vmcnt, lgkmcnt untouched
        __asm__ volatile("" ::: "memory");  // reads done before the next pass is written
      }
    }
    return;
  }

  // Epilogue.  Lane (r16, q) of block
  // (j, i) holds row m0 + 128 wave_m + 16 i + r16, columns n0 + 128 wave_n +
  // 16 j + 4 q + e, e = 0..3; a strip is A blocks 2s, 2s + 1 (32 rows).
  const float g_a = *a_gs;
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
  // kGates: a wave whose columns meet a gate range stages acc * alpha in
  // fp32, 16 rows x 64 columns at a time, in its strip buffer, applies the
  // gate functions in a rolled loop over it and stores element by element,
  // then leaves (no workgroup barrier follows); every other wave takes the
  // strip path below.
  if constexpr (kGates) {
    static_assert(kStripBytes >= 16 * 64 * 4, "fp32 half strip");
    if (cols_gated(cs, c_first, c_last)) {
      float* fs = reinterpret_cast<float*>(smem + STAGES * kStageBytes + wave * kStripBytes);
#pragma unroll
      for (int i = 0; i < FB; ++i)
#pragma unroll
        for (int hc = 0; hc < 2; ++hc) {
#pragma unroll
          for (int jl = 0; jl < 4; ++jl) {
            const int j = 4 * hc + jl, cl = 16 * j + 4 * q;  // column within the wave's 128
            const floatx4_t al4 = *reinterpret_cast<const floatx4_t*>(alpha_tab + cl);
            floatx4_t o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = acc[j][i][e] * al4[e];
            *reinterpret_cast<floatx4_t*>(fs + r16 * 64 + cl - 64 * hc) = o;
          }
          __asm__ volatile("" ::: "memory");  // other lanes' values are read below
          const int row0 = m0 + wave_m * WM + 16 * i, col0 = c_first + 64 * hc;
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
          __builtin_amdgcn_s_waitcnt(0xCF0F);  // expcnt(0): store data read before reuse
          __asm__ volatile("" ::: "memory");  // reads done before the next pass writes
        }
      return;
    }
  }
  const bool full_tile = vec_ok && m0 + BM <= M && n0 + BN <= N;
  uint8_t* strip = smem + STAGES * kStageBytes + wave * kStripBytes;
  constexpr int kChunksPerRow = kStripCols * kEsz / 16;
  constexpr int kChunkElems = 16 / kEsz;
  constexpr int kJPerPass = FB / kColPasses;
  floatx4_t al[FB];  // the lane's column scales
#pragma unroll
  for (int j = 0; j < FB; ++j) al[j] = *reinterpret_cast<const floatx4_t*>(alpha_tab + 16 * j + 4 * q);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int jp = 0; jp < kColPasses; ++jp) {  // columns [kStripCols jp, kStripCols (jp + 1)) of the wave
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int i = 2 * s + ii;
        uint8_t* rowp = strip + (16 * ii + r16) * kStripRow;
#pragma unroll
        for (int jl = 0; jl < kJPerPass; ++jl) {
          const int j = jp * kJPerPass + jl;
          const int col = 16 * jl + 4 * q;  // within the strip
          if constexpr (kOutBf16) {
            typedef __bf16 bf4_t __attribute__((ext_vector_type(4)));
            bf4_t o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (__bf16)(acc[j][i][e] * al[j][e]);
            *reinterpret_cast<bf4_t*>(rowp + col * kEsz) = o;
          } else {
            floatx4_t o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = acc[j][i][e] * al[j][e];
            *reinterpret_cast<floatx4_t*>(rowp + col * kEsz) = o;
          }
        }
      }
      const int grow0 = m0 + wave_m * WM + 32 * s;
      const int gcol0 = n0 + wave_n * WN + jp * kStripCols;
      constexpr int kQ = kStripRows * kChunksPerRow / 64;
      u32x4_t d[kQ];
#pragma unroll
      for (int qq = 0; qq < kQ; ++qq) {
        const int id = qq * 64 + lane;
        d[qq] = *reinterpret_cast<const u32x4_t*>(strip + (id / kChunksPerRow) * kStripRow + (id % kChunksPerRow) * 16);
      }
      if (full_tile) {
#pragma unroll
        for (int qq = 0; qq < kQ; ++qq) {
          const int id = qq * 64 + lane;
          const int r = id / kChunksPerRow, c = id % kChunksPerRow;
          out_t* dst = reinterpret_cast<out_t*>(y) + (int64_t)(grow0 + r) * ldy + gcol0 + c * kChunkElems;
          __builtin_nontemporal_store(d[qq], reinterpret_cast<u32x4_t*>(dst));
        }
      } else {
#pragma unroll
        for (int qq = 0; qq < kQ; ++qq) {
          const int id = qq * 64 + lane;
          const int r = id / kChunksPerRow, c = id % kChunksPerRow;
          const int grow = grow0 + r, gcol = gcol0 + c * kChunkElems;
          if (grow < M) {
            out_t* dst = reinterpret_cast<out_t*>(y) + (int64_t)grow * ldy + gcol;
            if (vec_ok && gcol + kChunkElems <= N) {
              __builtin_nontemporal_store(d[qq], reinterpret_cast<u32x4_t*>(dst));
            } else {
              const out_t* e = reinterpret_cast<const out_t*>(&d[qq]);
              for (int t = 0; t < kChunkElems; ++t)
                if (gcol + t < N) dst[t] = e[t];
            }
          }
        }
      }
      // the stores above must have read their data registers (expcnt)
      // before the next strip's LDS reads may reuse them
      __builtin_amdgcn_s_waitcnt(0xCF0F);  // expcnt(0); vmcnt, lgkmcnt untouched
      __asm__ volatile("" ::: "memory");  // the strip is read before it is written again
    }
  }
}

// Most K parts of a split tail tile.
constexpr int kMaxSplits = 8;

// Second kernel of a split tail: adds the K parts of each split tile in part
// order (fixed, so the output is deterministic) and writes the sums as the
// streaming epilogue does: y = sum * RN32(g_a g_w) of the column, then fp32
// or bf16 (RNE), with the GDN gate functions on gate columns (kGates), as
// the gated epilogue does.  The parts are row-major fp32 tiles [256 x 256]; block
// (t, y) covers rows 16y .. 16y + 15 of tail tile t, thread tid the columns
// 4 (tid % 64) .. + 3 of rows 16y + tid / 64 + 4r, r = 0..3.
template <bool kOutBf16, bool kGates>
__global__ __launch_bounds__(256) void split_tail_add_kernel(const SplitTail sp, const float* __restrict__ a_gs,
                                                             const ColScales cs, int M, int N,
                                                             void* __restrict__ y, int64_t ldy) {
  const int tid = threadIdx.x, c4 = tid & 63, r0 = 16 * (int)blockIdx.y + (tid >> 6);
  const int tiles_m = (M + 255) / 256, tiles_n = (N + 255) / 256;
  const bool vec_ok = ((uintptr_t)y % 16 == 0) && (ldy % 4 == 0);
  int tm, tn;
  tile_coords(sp.full + (int)blockIdx.x, tiles_m, tiles_n, tm, tn);
  // RN32(g_a g_i) of every column range, once per block
  __shared__ float alpha_of_range[kMaxModules];
  if (tid < cs.n) alpha_of_range[tid] = *a_gs * cs.gs[tid];
  const floatx4_t* base = reinterpret_cast<const floatx4_t*>(sp.part) + (size_t)blockIdx.x * sp.splits * (256 * 64);
  // every load first (up to kMaxSplits parts of 4 rows in flight), then the
  // sums in part order
  floatx4_t v[4][kMaxSplits];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr)
#pragma unroll
    for (int p = 0; p < kMaxSplits; ++p)
      if (p < sp.splits) v[rr][p] = base[(size_t)p * (256 * 64) + (r0 + 4 * rr) * 64 + c4];
  __syncthreads();  // the alpha table is written
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    floatx4_t sum = v[rr][0];
#pragma unroll
    for (int p = 1; p < kMaxSplits; ++p)
      if (p < sp.splits) sum += v[rr][p];
    const int row = tm * 256 + r0 + 4 * rr;
    const int col = tn * 256 + 4 * c4;
    if (row >= M || col >= N) continue;
    floatx4_t o;
#pragma unroll
    for (int t = 0; t < 4; ++t) o[t] = sum[t] * alpha_of_range[col_range(cs, min(col + t, N - 1))];
    if constexpr (kGates) {
#pragma unroll
      for (int t = 0; t < 4; ++t) o[t] = col_gate(cs, min(col + t, N - 1), o[t]);
    }
    if (vec_ok && col + 3 < N) {  // the 4 columns in one 8- or 16-byte store
      if constexpr (kOutBf16) {
        typedef __bf16 bf4_t __attribute__((ext_vector_type(4)));
        *reinterpret_cast<bf4_t*>(reinterpret_cast<__bf16*>(y) + (int64_t)row * ldy + col) =
            bf4_t{(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
      } else {
        *reinterpret_cast<floatx4_t*>(reinterpret_cast<float*>(y) + (int64_t)row * ldy + col) = o;
      }
      continue;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (col + t >= N) break;
      if constexpr (kOutBf16)
        reinterpret_cast<__bf16*>(y)[(int64_t)row * ldy + col + t] = (__bf16)o[t];
      else
        reinterpret_cast<float*>(y)[(int64_t)row * ldy + col + t] = o[t];
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
//  * v_mfma_f32_16x16x32_f16 wants lane L to hold row L % 16 of its 16-row
//    block.  The code loads deliver that layout directly: load h (0 or 1) of
//    a block gives lane L row L % 16, 16-byte chunk 2 (L / 16) + h of the
//    tile, so a lane group g of 16 lanes holds chunks 2g and 2g + 1.  The
//    two loads of a block read the halves of the same 128-byte row pieces.
//    (Loads of 8 rows x 128 contiguous bytes, turned into this layout with
//    two DPP row shifts per dword, took 60 more VALU per tile and measured
//    1-4% slower at every M.)  A is loaded the same way (it stays in L2).
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

template <int MB16, int NB, int D, int kXIn, bool kPeel>
__global__ __launch_bounds__(64 * kDecodeWaves) void gemm_decode_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_gs,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, const ColScales cs,
    int M, int N, int K, void* __restrict__ y, int64_t ldy, bool out_bf16, int nt_max,
    const void* __restrict__ x, int64_t ldx) {
  constexpr int NW = 16 * NB;  // weight rows per workgroup
  constexpr int MA = 16 * MB16;
  constexpr int kTileBytes = 128, kTileScales = 16;  // per row, per 256-value tile
  constexpr int kLoads = 2 * NB + (kXIn ? 0 : 2 * MB16);  // code loads per tile
  constexpr int kVmPerTile = kLoads + (kXIn ? 2 : 0);      // vector loads per tile (kXIn: + 2 of x)
  static_assert(kXIn == 0 || (kXIn == 1 && MB16 == 1), "in-kernel quantization: bf16, M <= kFusedRows");
  static_assert(D * kVmPerTile < 64, "vmcnt range");
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
  // load i: block i / 2, all 16 rows (lane L: row L % 16) x 16-byte chunk
  // 2 (L / 16) + i % 2 of the tile (the MFMA operand layout)
#pragma unroll
  for (int i = 0; i < 2 * NB; ++i)
    w_off[i] = (uint32_t)(n0 + 16 * (i / 2) + (lane & 15)) * row_bytes + (uint32_t)(2 * (lane >> 4) + i % 2) * 16;
#pragma unroll
  for (int i = 0; i < 2 * MB16; ++i)
    a_off[i] = (uint32_t)(16 * (i / 2) + (lane & 15)) * row_bytes + (uint32_t)(2 * (lane >> 4) + i % 2) * 16;

  struct Tile {
    u32x4_t x[kXIn ? 2 : 1];  // kXIn: the lane's 16 bf16 values
    u32x4_t w[2 * NB];
    u32x4_t a[2 * MB16];
  };
  // Tile t0 + t of this wave.  The tile's offset in the rows is the
  // wave-uniform SGPR offset of the loads, so the per-lane offsets stay
  // fixed and no vector instruction addresses a tile.  Tiles past the wave's
  // range (t >= nt) are read through resources of size 0 (a uniform select
  // of SGPRs): the loads return zeros without touching memory, and the zero
  // tile adds nothing to the sums.  That keeps the main loop branch-free,
  // so the compiler can wait for each tile individually instead of draining
  // every load in flight.
  const __amdgpu_buffer_rsrc_t rw_none = make_rsrc(w_codes, 0), ra_none = make_rsrc(a_codes, 0);
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
    const __amdgpu_buffer_rsrc_t rwt = ok ? rw : rw_none;
#pragma unroll
    for (int i = 0; i < 2 * NB; ++i) T.w[i] = __builtin_amdgcn_raw_buffer_load_b128(rwt, w_off[i], kc, 0);
    if constexpr (kXIn == 0) {
      const __amdgpu_buffer_rsrc_t rat = ok ? ra : ra_none;
#pragma unroll
      for (int i = 0; i < 2 * MB16; ++i) T.a[i] = __builtin_amdgcn_raw_buffer_load_b128(rat, a_off[i], kc, 0);
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
    // the four block scales as exact fp16 values: pair c holds the scales of
    // chunk c (bytes 2c, 2c + 1 of the dword)
    half2_t wsp[NB][2], asp[MB16][2];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      wsp[j][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wsd[j], 1.0f, false);
      wsp[j][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wsd[j], 1.0f, true);
    }
#pragma unroll
    for (int b = 0; b < MB16; ++b) {
      asp[b][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(asd[b], 1.0f, false);
      asp[b][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(asd[b], 1.0f, true);
    }
    // operands: chunks 2g (index 0) and 2g + 1 (index 1) of the lane's row
    u32x4_t wr[NB][2], ar[MB16][2];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      wr[j][0] = T.w[2 * j];
      wr[j][1] = T.w[2 * j + 1];
    }
    if constexpr (kXIn == 0) {
#pragma unroll
      for (int b = 0; b < MB16; ++b) {
        ar[b][0] = T.a[2 * b];
        ar[b][1] = T.a[2 * b + 1];
      }
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
      const int c = s >> 2, dw = s & 3;
#pragma unroll
      for (int b = 0; b < MB16; ++b) av[slot][b] = dequant8_sel(ar[b][c][dw], asp[b][c], dw >> 1);
#pragma unroll
      for (int j = 0; j < NB; ++j) wv[slot][j] = dequant8_sel(wr[j][c][dw], wsp[j][c], dw >> 1);
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
    // kPeel (every wave has at least D tiles): the loop's first pass is
    // unconditional, so the compiler has no guarded block to sink the ring's
    // loads into and issues all D tiles before the wait; since vector memory
    // operations complete in order, a count of the ring's loads then covers
    // the copies, and tiles 1 .. D - 1 stay in flight while tile 0 is
    // computed.  (With the first round inside the loop, the compiler moved
    // tile 1's loads past the wait into the loop's preheader, where a count
    // no longer covered the copies; a CPU test checks the compiled code.)
    // Otherwise the wait drains every load in flight.
    if constexpr (kPeel) {
      wait_vmcnt<D * kVmPerTile>();
    } else {
      wait_vmcnt<0>();
    }
    __asm__ volatile("" ::: "memory");  // no LDS read moves above the wait
    const int n_full = nt / D;
    // kPeel: the first pass of the loop is unconditional (n_full >= 1), so
    // the compiler emits no guard branch around it
    for (int it = 0; kPeel ? (it == 0 || it < n_full) : it < n_full; ++it) {
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
    mfma_drain();
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
  // every wave has at least (K / 256) / kDecodeWaves tiles
  const int nt_min = (int)((K / 256) / kDecodeWaves);
#define NVFP4_DECODE_KERNEL(MB, NBB, DD, PEEL)                                                                      \
  do {                                                                                                               \
    const size_t lds = decode_lds_bytes<MB, NBB, kXIn>(nt_max);                                                      \
    if (lds > kDecodeMaxLds || !allow_lds((const void*)gemm_decode_kernel<MB, NBB, DD, kXIn, PEEL>, lds))          \
      return false;                                                                                                  \
    gemm_decode_kernel<MB, NBB, DD, kXIn, PEEL><<<grid, block, lds, stream>>>(                                      \
        a_codes, a_scales, a_gs, w_codes, w_scales, cs, m, n, k, y, ldy, out_bf16, nt_max, x, ldx);                  \
    *err = hipGetLastError();                                                                                        \
    return true;                                                                                                     \
  } while (0)
  // The counted prologue wait (kPeel) for one 16-row block of A only: at
  // M <= 16 it measured 0.4 us faster at N = 12384, K = 5120 (11.0 against
  // 11.4 us at M = 1), at M = 32-64 1-4% slower.
#define NVFP4_DECODE_NB(MB, NBB, DD)                                            \
  do {                                                                          \
    if constexpr (MB == 1) {                                                    \
      if (nt_min >= DD) NVFP4_DECODE_KERNEL(MB, NBB, DD, true);                 \
    }                                                                           \
    NVFP4_DECODE_KERNEL(MB, NBB, DD, false);                                    \
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
#undef NVFP4_DECODE_KERNEL
  return false;
}

// Workgroups in one round of the large-tile kernel: one per CU.
constexpr int kRound = 256;

// Whether the large-tile kernel takes the shape (apart from pointer
// alignment): K in whole 128-value steps, 32-bit buffer offsets, and at
// least one full round of tiles.
bool stream_shape(int64_t M, int64_t N, int64_t K) {
  const bool fits32 = M * (K / 2) < ((int64_t)1 << 31) && N * (K / 2) < ((int64_t)1 << 31);
  return K % kBK == 0 && fits32 && ((M + 255) / 256) * ((N + 255) / 256) >= kRound;
}

}  // namespace

SplitTail gemm_split_plan(int64_t M, int64_t N, int64_t K) {
  SplitTail sp{};
  if (M <= 0 || N <= 0 || !stream_shape(M, N, K)) return sp;
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  const int64_t tail = tiles % kRound;
  // Split only a last round at most a quarter full, into parts of at least
  // 4 K steps, at most kMaxSplits of them (the partial sums are 256 KiB per
  // part and are written and read once more), filling at most one round.
  if (tail == 0 || tail > kRound / 4) return sp;
  const int splits = (int)std::min<int64_t>(std::min<int64_t>(kRound / tail, kMaxSplits), (K / kBK) / 4);
  if (splits < 2) return sp;
  sp.full = (int)(tiles - tail);
  sp.tail = (int)tail;
  sp.splits = splits;
  return sp;
}

size_t gemm_split_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const SplitTail sp = gemm_split_plan(M, N, K);
  return (size_t)sp.tail * (size_t)sp.splits * (64 * 256 * sizeof(floatx4_t));
}

namespace {

// The large-tile launch, with the tail split when `sp.splits` > 0.
template <bool kOutBf16, bool kGates>
hipError_t launch_stream(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
                         const uint8_t* w_codes, const uint8_t* w_scales, const ColScales& cs, int M, int N,
                         int K, void* y, int64_t ldy, const SplitTail& sp, hipStream_t stream) {
  constexpr int kStages = 3;
  const int64_t tiles = ((int64_t)(M + 255) / 256) * ((N + 255) / 256);
  // whole tiles (all of them without a split), then the K parts of the tail
  // tiles, then their sums: three launches in stream order
  gemm_stream16_kernel<kStages, kOutBf16, kGates, false>
      <<<dim3((unsigned)(sp.splits > 0 ? sp.full : tiles)), dim3(256), 0, stream>>>(
          a_codes, a_scales, a_gs, w_codes, w_scales, cs, M, N, K, y, ldy, sp, SwigluOut{});
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || sp.splits == 0) return err;
  gemm_stream16_kernel<kStages, false, false, true><<<dim3((unsigned)(sp.tail * sp.splits)), dim3(256), 0, stream>>>(
      a_codes, a_scales, a_gs, w_codes, w_scales, cs, M, N, K, nullptr, 0, sp, SwigluOut{});
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  split_tail_add_kernel<kOutBf16, kGates><<<dim3((unsigned)sp.tail, 16), dim3(256), 0, stream>>>(sp, a_gs, cs, M, N, y,
                                                                                                  ldy);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
                       const uint8_t* w_codes, const uint8_t* w_scales, const ColScales& cs,
                       int64_t M, int64_t N, int64_t K, void* y, bool out_bf16, int64_t ldy,
                       hipStream_t stream, void* workspace, size_t workspace_bytes) {
  const bool aligned = (K % kBK == 0) && ((uintptr_t)a_codes % 16 == 0) && ((uintptr_t)w_codes % 16 == 0) &&
                       ((uintptr_t)a_scales % 8 == 0) && ((uintptr_t)w_scales % 8 == 0);
  if (aligned && stream_shape(M, N, K)) {
    const bool gates = cs.decay_hi > cs.decay_lo || cs.write_hi > cs.write_lo;
    SplitTail sp{};
    if (workspace && (uintptr_t)workspace % 16 == 0) {
      sp = gemm_split_plan(M, N, K);
      if (workspace_bytes < gemm_split_workspace_bytes(M, N, K)) sp = SplitTail{};
      sp.part = static_cast<float*>(workspace);
    }
    const int m = (int)M, n = (int)N, k = (int)K;
    if (out_bf16) {
      if (gates) return launch_stream<true, true>(a_codes, a_scales, a_gs, w_codes, w_scales, cs, m, n, k, y, ldy, sp, stream);
      return launch_stream<true, false>(a_codes, a_scales, a_gs, w_codes, w_scales, cs, m, n, k, y, ldy, sp, stream);
    }
    if (gates) return launch_stream<false, true>(a_codes, a_scales, a_gs, w_codes, w_scales, cs, m, n, k, y, ldy, sp, stream);
    return launch_stream<false, false>(a_codes, a_scales, a_gs, w_codes, w_scales, cs, m, n, k, y, ldy, sp, stream);
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
  gemm_stream16_kernel<3, true, false, false, true><<<dim3((unsigned)tiles), dim3(256), 0, stream>>>(
      a_codes, a_scales, a_gs, w_codes, w_scales, cs, (int)M, (int)(2 * F), (int)K, nullptr, 0, SplitTail{}, out);
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
