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
#include <type_traits>

#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

constexpr int kBK = 128;              // K values per main-loop step
constexpr int kRowBytes = kBK / 2;    // 64 code bytes per row per step
constexpr int kLdsRow = kRowBytes + 16;  // padded LDS row stride: conflict-free 16-byte reads
constexpr int kScaleBytes = kBK / 16;    // 8 scale bytes per row per step

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
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, const float* __restrict__ w_gs,
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

  // epilogue: y = acc * RN32(g_a g_w)
  const float alpha = (*a_gs) * (*w_gs);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wave_n * WN + j * 32 + r32;
      if (col >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wave_m * WM + i * 32 + (v >> 2) * 8 + half * 4 + (v & 3);
        if (row < M) {
          const float o = acc[i][j][v] * alpha;
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
template <int STAGES, bool kOutBf16>
__global__ __launch_bounds__(256) void gemm_stream_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_gs,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, const float* __restrict__ w_gs,
    int M, int N, int K, void* __restrict__ y, int64_t ldy) {
  constexpr int BM = 256, BN = 256, WM = 128, WN = 128, FM = 4, FN = 4;
  constexpr int kCodeBytes = BM * kRowBytes;          // 16 KiB per operand per stage
  constexpr int kStageScaleBytes = BM * kScaleBytes;  // 2 KiB per operand per stage
  constexpr int kStageBytes = 2 * kCodeBytes + 2 * kStageScaleBytes;
  constexpr int kLoadsPerStage = 12;                  // vector-memory instructions per wave per stage
  using out_t = typename std::conditional<kOutBf16, __bf16, float>::type;
  constexpr int kEsz = sizeof(out_t);
  constexpr int kStripRows = 16;                      // output rows staged per pass
  constexpr int kStripRow = WN * kEsz + 16;           // staged row bytes (+16 against bank conflicts)
  constexpr int kStripBytes = kStripRows * kStripRow;
  static_assert(STAGES >= 3, "ring depth");
  static_assert((STAGES - 1) * kLoadsPerStage < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * kStageBytes + 4 * kStripBytes];
  uint8_t* const ring = smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int wave_m = wave >> 1, wave_n = wave & 1;
  const int r32 = lane & 31, half = lane >> 5;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int64_t row_bytes = K / 2, srow_bytes = K / 16;
  const int ksteps = K / kBK;
  const float alpha = (*a_gs) * (*w_gs);
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
  auto set_sources = [&](int m0, int n0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wave * 64 + 16 * i + (lane >> 2);
      const int chunk = (lane & 3) ^ chunk_swizzle(row);
      a_off[i] = (uint32_t)min(m0 + row, M - 1) * (uint32_t)row_bytes + chunk * 16;
      w_off[i] = (uint32_t)min(n0 + row, N - 1) * (uint32_t)row_bytes + chunk * 16;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = wave * 64 + 32 * i + (lane >> 1);
      as_off[i] = (uint32_t)min(m0 + row, M - 1) * (uint32_t)srow_bytes + (lane & 1) * 4;
      ws_off[i] = (uint32_t)min(n0 + row, N - 1) * (uint32_t)srow_bytes + (lane & 1) * 4;
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
  auto mfma_step = [&](int cur) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int i = 0; i < FM; ++i)
        acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[cur][j], af[cur][i], acc[j][i], 0, 0, 0);
  };
  // Issue order inside one MFMA step: each MFMA is followed by 4 VALU
  // (dequantization of the next step) and optionally one copy and/or LDS read.
  auto schedule = [&](int n_vmem, int n_ds) {
#pragma unroll
    for (int g = 0; g < FM * FN; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);    // VALU
      if (g < n_vmem) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read (copy)
      if (g < n_ds) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // DS read
    }
  };

  // first K tile: wait for its copies, then read its first half + scales
  wait_vmcnt<(STAGES - 1) * kLoadsPerStage>();
  __builtin_amdgcn_s_barrier();
  read_half(0, 0, true);

  for (int ks = 0; ks < ksteps; ++ks) {
    const int slot = ks % STAGES;
#pragma unroll
    for (int i = 0; i < FM; ++i) a_sc[i] = a_sc_next[i];
#pragma unroll
    for (int j = 0; j < FN; ++j) w_sc[j] = w_sc_next[j];
    // phase 1: MFMA steps 0..3 from half 0 while half 1 of this K tile is read
    dequant_step(0, 0);
    read_half(slot, 1, false);
    dequant_step(1, 1);
    mfma_step(0);
    schedule(0, FM + FN);
#pragma unroll
    for (int kk = 1; kk < 4; ++kk) {
      dequant_step(kk + 1, (kk + 1) & 1);
      mfma_step(kk & 1);
      schedule(0, 0);
    }
    // mid-tile: K tile ks+1 has landed (own copies + barrier); the slot just
    // read is refilled with K tile ks+STAGES (clamped)
    wait_vmcnt<(STAGES - 2) * kLoadsPerStage>();
    // a bare s_barrier: __syncthreads() would also wait for every copy in
    // flight and drain the ring
    __builtin_amdgcn_s_barrier();
    issue_stage(min(ks + STAGES, ksteps - 1), slot);
    read_half((ks + 1) % STAGES, 0, true);
    // phase 2: MFMA steps 4..7 from half 1 while the next K tile's half 0 is read
    dequant_step(5, 1);
    mfma_step(0);
    schedule(kLoadsPerStage, FM * FN);
#pragma unroll
    for (int kk = 5; kk < 8; ++kk) {
      if (kk + 1 < 8) dequant_step(kk + 1, (kk + 1) & 1);
      mfma_step(kk & 1);
      if (kk + 1 < 8) schedule(0, 0);
    }
  }
  wait_vmcnt<0>();  // the repeated copies past the last K tile
  __syncthreads();  // every wave is done with the ring

  {
    // Epilogue.  Lane (r32, half) of block (j, i) holds, for output row
    // m = m0 + 128 wave_m + 32 i + r32, the columns n0 + 128 wave_n + 32 j +
    // 8 (v / 4) + 4 half + (v % 4), v = 0..15: four consecutive columns per
    // group of 4 accumulators.  Rows go through LDS in strips of 16.
    uint8_t* strip = smem + STAGES * kStageBytes + wave * kStripBytes;
    constexpr int kChunksPerRow = WN * kEsz / 16;
    constexpr int kChunkElems = 16 / kEsz;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {      // rows r32 in [16 sub, 16 sub + 16)
        if ((r32 >> 4) == sub) {
          uint8_t* rowp = strip + (r32 & 15) * kStripRow;
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int col = j * 32 + g * 8 + half * 4;
              if constexpr (kOutBf16) {
                typedef __bf16 bf4_t __attribute__((ext_vector_type(4)));
                bf4_t o;
#pragma unroll
                for (int t = 0; t < 4; ++t) o[t] = (__bf16)(acc[j][i][4 * g + t] * alpha);
                *reinterpret_cast<bf4_t*>(rowp + col * kEsz) = o;
              } else {
                floatx4_t o;
#pragma unroll
                for (int t = 0; t < 4; ++t) o[t] = acc[j][i][4 * g + t] * alpha;
                *reinterpret_cast<floatx4_t*>(rowp + col * kEsz) = o;
              }
            }
        }
        const int grow0 = m0 + wave_m * WM + i * 32 + sub * 16;
        const int gcol0 = n0 + wave_n * WN;
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

// Decode kernel (M <= 64): bound by the weight stream, N x K x 0.5625 bytes.
//
// A workgroup owns 48 weight rows (three 16-row MFMA blocks; 256 workgroups
// cover N = 12288, one per CU) and all M rows of A.  Its 4 waves split K
// into quarters, and each wave streams its quarter of W and of A through a
// private ring of R K tiles in LDS with direct global->LDS copies, R tiles
// ahead (>= 100 KB in flight per CU, enough to cover HBM latency at full
// bandwidth).  A wave reads only its own ring, so no barrier is needed
// inside the loop; a wave's copies complete in issue order, so one vmcnt
// wait per K tile suffices.  MFMA 16x16x32 f16 with W as the "A" operand:
// each lane ends up with 4 consecutive output columns of one row.  The four
// partial sums are added through LDS in a fixed order (deterministic).
// MB16 = number of 16-row blocks of A (1, 2 or 4).
template <int MB16, int R, bool kOutBf16>
__global__ __launch_bounds__(256) void gemm_decode_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_gs,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, const float* __restrict__ w_gs,
    int M, int N, int K, void* __restrict__ y, int64_t ldy) {
  constexpr int NW = 48;                           // weight rows per workgroup
  constexpr int MA = 16 * MB16;                    // A rows per workgroup (padded)
  constexpr int kWCode = NW * kRowBytes;           // 3072 B
  constexpr int kWScale = NW * kScaleBytes;        // 384 B
  constexpr int kACode = MA * kRowBytes;
  constexpr int kAScale = MA * kScaleBytes;
  constexpr int kSlot = kWCode + kWScale + kACode + kAScale;
  constexpr int kWScaleInstr = (kWScale + 255) / 256;
  constexpr int kAScaleInstr = (kAScale + 255) / 256;
  constexpr int kPerSlot = 3 + kWScaleInstr + MB16 + kAScaleInstr;  // copy instructions per K tile
  static_assert((R - 1) * kPerSlot < 64, "vmcnt range");
  static_assert(4 * R * kSlot <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * R * kSlot];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int r16 = lane & 15, kg = lane >> 4;
  const int n0 = blockIdx.x * NW;
  const int64_t row_bytes = K / 2, srow_bytes = K / 16;
  const int ksteps = K / kBK;
  const int kq0 = (ksteps * wave) / 4, nk = (ksteps * (wave + 1)) / 4 - kq0;
  uint8_t* const ring = smem + wave * R * kSlot;

  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w_codes, (int64_t)N * row_bytes);
  const __amdgpu_buffer_rsrc_t rws = make_rsrc(w_scales, (int64_t)N * srow_bytes);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_codes, (int64_t)M * row_bytes);
  const __amdgpu_buffer_rsrc_t ras = make_rsrc(a_scales, (int64_t)M * srow_bytes);
  // per-lane copy offsets (K tile 0 of the workgroup's rows)
  uint32_t w_off[3], a_off[MB16], ws_off[kWScaleInstr], as_off[kAScaleInstr];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int row = 16 * i + (lane >> 2);
    w_off[i] = (uint32_t)min(n0 + row, N - 1) * (uint32_t)row_bytes + (((lane & 3) ^ chunk_swizzle(row)) * 16);
  }
#pragma unroll
  for (int i = 0; i < MB16; ++i) {
    const int row = 16 * i + (lane >> 2);
    a_off[i] = (uint32_t)min(row, M - 1) * (uint32_t)row_bytes + (((lane & 3) ^ chunk_swizzle(row)) * 16);
  }
#pragma unroll
  for (int i = 0; i < kWScaleInstr; ++i) {
    const int d = 64 * i + lane;  // dword index: row d / 2, half d % 2
    ws_off[i] = (uint32_t)min(n0 + d / 2, N - 1) * (uint32_t)srow_bytes + (d & 1) * 4;
  }
#pragma unroll
  for (int i = 0; i < kAScaleInstr; ++i) {
    const int d = 64 * i + lane;
    as_off[i] = (uint32_t)min(d / 2, M - 1) * (uint32_t)srow_bytes + (d & 1) * 4;
  }
  auto issue = [&](int t, int slot) {  // K tile kq0 + t of this wave into ring slot
    uint8_t* st = ring + slot * kSlot;
    const uint32_t kc = (uint32_t)(kq0 + t) * kRowBytes, ksc = (uint32_t)(kq0 + t) * kScaleBytes;
#pragma unroll
    for (int i = 0; i < 3; ++i) lds_copy16(rw, w_off[i], kc, st + i * 1024);
#pragma unroll
    for (int i = 0; i < kWScaleInstr; ++i)
      if (64 * i + lane < kWScale / 4) lds_copy4(rws, ws_off[i], ksc, st + kWCode + i * 256);
#pragma unroll
    for (int i = 0; i < MB16; ++i) lds_copy16(ra, a_off[i], kc, st + kWCode + kWScale + i * 1024);
#pragma unroll
    for (int i = 0; i < kAScaleInstr; ++i)
      if (64 * i + lane < kAScale / 4) lds_copy4(ras, as_off[i], ksc, st + kWCode + kWScale + kACode + i * 256);
  };

  floatx4_t acc[3][MB16];
#pragma unroll
  for (int j = 0; j < 3; ++j)
#pragma unroll
    for (int b = 0; b < MB16; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[j][b][v] = 0.0f;

  if (nk > 0) {
#pragma unroll
    for (int t = 0; t < R; ++t) issue(min(t, nk - 1), t);
    for (int t0 = 0; t0 < nk; t0 += R) {
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int t = t0 + u;
        if (t < nk) {
          wait_vmcnt<(R - 1) * kPerSlot>();
          const uint8_t* st = ring + u * kSlot;
          u32x4_t wc[3], ac[MB16];
          uint32_t wsd[3], asd[MB16];
#pragma unroll
          for (int j = 0; j < 3; ++j) {
            const int row = 16 * j + r16;
            wc[j] = *reinterpret_cast<const u32x4_t*>(st + row * kRowBytes + 16 * (kg ^ chunk_swizzle(row)));
            wsd[j] = *reinterpret_cast<const uint32_t*>(st + kWCode + row * kScaleBytes + 4 * (kg >> 1));
          }
#pragma unroll
          for (int b = 0; b < MB16; ++b) {
            const int row = 16 * b + r16;
            ac[b] = *reinterpret_cast<const u32x4_t*>(st + kWCode + kWScale + row * kRowBytes + 16 * (kg ^ chunk_swizzle(row)));
            asd[b] = *reinterpret_cast<const uint32_t*>(st + kWCode + kWScale + kACode + row * kScaleBytes + 4 * (kg >> 1));
          }
          // Operands of step s+1 are dequantized into the other half of a
          // double buffer while the MFMAs of step s run, one MFMA then a few
          // VALU at a time.  An MFMA's source registers are therefore never
          // rewritten until at least one more MFMA has issued: a VALU write
          // to them right behind a 16x16x32 MFMA was seen to corrupt the
          // MFMA's input for the upper 8 rows of its A operand.
          half8_t wv[2][3], av[2][MB16];
          auto deq = [&](int s, int slot_) {
            const int sb = 8 * (2 * (kg & 1) + (s >> 1));  // this step's scale byte in the lane's dword
#pragma unroll
            for (int b = 0; b < MB16; ++b) av[slot_][b] = dequant8(ac[b][s], scale_pair((asd[b] >> sb) & 0xFFu));
#pragma unroll
            for (int j = 0; j < 3; ++j) wv[slot_][j] = dequant8(wc[j][s], scale_pair((wsd[j] >> sb) & 0xFFu));
          };
          deq(0, 0);
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            if (s + 1 < 4) deq(s + 1, (s + 1) & 1);
#pragma unroll
            for (int j = 0; j < 3; ++j)
#pragma unroll
              for (int b = 0; b < MB16; ++b)
                acc[j][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv[s & 1][j], av[s & 1][b], acc[j][b], 0, 0, 0);
            if (s + 1 < 4) {
#pragma unroll
              for (int g = 0; g < 3 * MB16; ++g) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                          // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, (8 * (3 + MB16) + 3 * MB16 - 1) / (3 * MB16), 0);  // VALU
              }
            }
          }
          // this slot's LDS reads are complete (their data fed the MFMAs);
          // refill it with K tile t + R (repeating the last one past the end)
          __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
          issue(min(t + R, nk - 1), u);
        }
      }
    }
  }
  wait_vmcnt<0>();
  __syncthreads();

  // fixed-order sum of the 4 K quarters through LDS (the ring is free now)
  float* red = reinterpret_cast<float*>(smem);  // [3 waves][3][MB16][4][64]
  if (wave > 0) {
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
      for (int b = 0; b < MB16; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[(((wave - 1) * 3 + j) * MB16 + b) * 256 + v * 64 + lane] = acc[j][b][v];
  }
  __syncthreads();
  if (wave == 0) {
    const float alpha = (*a_gs) * (*w_gs);
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
      for (int b = 0; b < MB16; ++b) {
        const int m = 16 * b + r16;
        const int n = n0 + 16 * j + 4 * kg;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float t = acc[j][b][v];
#pragma unroll
          for (int w = 0; w < 3; ++w) t += red[((w * 3 + j) * MB16 + b) * 256 + v * 64 + lane];
          if (m < M && n + v < N) {
            const float o = t * alpha;
            if constexpr (kOutBf16) reinterpret_cast<__bf16*>(y)[(int64_t)m * ldy + n + v] = (__bf16)o;
            else reinterpret_cast<float*>(y)[(int64_t)m * ldy + n + v] = o;
          }
        }
      }
  }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_tiles(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
                        const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gs, int64_t M,
                        int64_t N, int64_t K, void* y, bool out_bf16, int64_t ldy, bool aligned,
                        hipStream_t stream) {
  constexpr int kThreads = (BM / WM) * (BN / WN) * 64;
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const dim3 grid((unsigned)tiles), block(kThreads);
  const int m = (int)M, n = (int)N, k = (int)K;
  if (aligned) {
    if (out_bf16)
      gemm_kernel<BM, BN, WM, WN, true, true><<<grid, block, 0, stream>>>(a_codes, a_scales, a_gs, w_codes, w_scales, w_gs, m, n, k, y, ldy);
    else
      gemm_kernel<BM, BN, WM, WN, true, false><<<grid, block, 0, stream>>>(a_codes, a_scales, a_gs, w_codes, w_scales, w_gs, m, n, k, y, ldy);
  } else {
    if (out_bf16)
      gemm_kernel<BM, BN, WM, WN, false, true><<<grid, block, 0, stream>>>(a_codes, a_scales, a_gs, w_codes, w_scales, w_gs, m, n, k, y, ldy);
    else
      gemm_kernel<BM, BN, WM, WN, false, false><<<grid, block, 0, stream>>>(a_codes, a_scales, a_gs, w_codes, w_scales, w_gs, m, n, k, y, ldy);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
                       const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gs,
                       int64_t M, int64_t N, int64_t K, void* y, bool out_bf16, int64_t ldy,
                       hipStream_t stream) {
  const bool aligned = (K % kBK == 0) && ((uintptr_t)a_codes % 16 == 0) && ((uintptr_t)w_codes % 16 == 0) &&
                       ((uintptr_t)a_scales % 8 == 0) && ((uintptr_t)w_scales % 8 == 0);
  const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
  const bool fits32 = M * (K / 2) < ((int64_t)1 << 31) && N * (K / 2) < ((int64_t)1 << 31);
  if (aligned && fits32 && big_tiles >= 256) {
    constexpr int kStages = 3;
    const dim3 grid((unsigned)big_tiles), block(256);
    if (out_bf16)
      gemm_stream_kernel<kStages, true><<<grid, block, 0, stream>>>(a_codes, a_scales, a_gs, w_codes, w_scales, w_gs,
                                                                   (int)M, (int)N, (int)K, y, ldy);
    else
      gemm_stream_kernel<kStages, false><<<grid, block, 0, stream>>>(a_codes, a_scales, a_gs, w_codes, w_scales, w_gs,
                                                                    (int)M, (int)N, (int)K, y, ldy);
    return hipGetLastError();
  }
  if (aligned && fits32 && M <= 64) {
    const dim3 grid((unsigned)((N + 47) / 48)), block(256);
    const int m = (int)M, n = (int)N, k = (int)K;
#define NVFP4_DECODE(MB, RR)                                                                                  \
  do {                                                                                                         \
    if (out_bf16)                                                                                              \
      gemm_decode_kernel<MB, RR, true><<<grid, block, 0, stream>>>(a_codes, a_scales, a_gs, w_codes, w_scales, \
                                                                   w_gs, m, n, k, y, ldy);                     \
    else                                                                                                       \
      gemm_decode_kernel<MB, RR, false><<<grid, block, 0, stream>>>(a_codes, a_scales, a_gs, w_codes, w_scales, \
                                                                    w_gs, m, n, k, y, ldy);                    \
  } while (0)
    if (M <= 16) NVFP4_DECODE(1, 8);
    else if (M <= 32) NVFP4_DECODE(2, 6);
    else NVFP4_DECODE(4, 4);
#undef NVFP4_DECODE
    return hipGetLastError();
  }
  return launch_tiles<128, 128, 64, 64>(a_codes, a_scales, a_gs, w_codes, w_scales, w_gs, M, N, K, y,
                                        out_bf16, ldy, aligned, stream);
}

}  // namespace nvfp4
