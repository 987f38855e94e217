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

#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      half8_t af[FM], wf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const uint32_t c = a_raw[i][kk >> 2][kk & 3];
        af[i] = dequant8(c, scale_pair((a_sc[i] >> (8 * (kk >> 1))) & 0xFFu));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const uint32_t c = w_raw[j][kk >> 2][kk & 3];
        wf[j] = dequant8(c, scale_pair((w_sc[j] >> (8 * (kk >> 1))) & 0xFFu));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], wf[j], acc[i][j], 0, 0, 0);
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
  if (big_tiles >= 512) {
    return launch_tiles<256, 256, 128, 128>(a_codes, a_scales, a_gs, w_codes, w_scales, w_gs, M, N, K, y,
                                            out_bf16, ldy, aligned, stream);
  }
  return launch_tiles<128, 128, 64, 64>(a_codes, a_scales, a_gs, w_codes, w_scales, w_gs, M, N, K, y,
                                        out_bf16, ldy, aligned, stream);
}

}  // namespace nvfp4
