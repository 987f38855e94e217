// Gated DeltaNet recurrence for gfx950, fp32 state.
//
// The recurrence of the picx.dev summary page ("Introduction and Theoretical
// Foundation" > "Gated DeltaNet Mechanics"), as printed there: per value head
// a state S (d_k x d_v), and per token
//     u   = S_{t-1}^T k
//     S_t = alpha_t S_{t-1} + beta_t k (v_t - u)^T
//     o_t = S_t^T q / sqrt(d_k)
// with alpha_t = exp(g_t) (g the log-space decay gate) and beta_t the write
// strength.  q and k are taken L2-normalized (per head), so that the update
// operator alpha I - beta k k^T has norm <= 1 and the state cannot grow.
//
// Inputs are the projection outputs of a token, one row per token: q, k, v,
// g and beta at given column offsets of an fp32 row (the fused GDN
// in-projection with its gate epilogue writes exactly such rows).  Value
// head h reads q/k head h * n_qk / n_v.  d_k = d_v = 128.
//
// The columns of S are independent: column j needs only its own
// u_j = S[:, j]^T k, its own update S[:, j] += k beta (v_j - u_j) and gives
// o_j = S[:, j]^T q.  So the state is split by columns over workgroups that
// never exchange anything, and the 128 rows of a column over kParts
// consecutive lanes of one wave (128 / kParts rows each, in registers).  The
// row sums are DPP sums over those lanes: a token needs no LDS access and no
// barrier, and the heads' columns keep the whole chip busy.
//  * kParts = 16 (8 rows per lane) and 16 columns per workgroup (4 waves):
//    8 workgroups per value head, 256 for 32 heads.
//  * When the squared Frobenius norm of every S_t is asked for, a workgroup
//    takes a whole head (kParts = 8, 128 columns, 16 waves); the waves'
//    shares of the norm meet in LDS and are added once per 64 tokens.
// Each lane loads its rows of k and q (and its v) for every token, kAhead
// tokens ahead, in a ring of register slots indexed at compile time.  The
// per-token scalars 1 / |k|, 1 / (|q| sqrt(d)) and alpha, the same for the
// whole head, are formed once per chunk of 64 tokens.  Loads and stores go
// through buffer resources so that none sits in a branch, and snapshots
// split the tokens into segments, so that the compiler keeps the ring's
// loads in flight across tokens.
// (One workgroup of 1024 threads per head, with the row parts of a column
// spread over waves and summed through LDS, took 1.28 us per token with two
// barriers; this form takes 0.16-0.23 us per token on 32 heads.)
#include <hip/hip_runtime.h>

#include <cstdint>

#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

constexpr int kD = 128;       // head dimension (d_k = d_v)
constexpr float kNormEps = 1e-6f;

template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask, 0xF, false));
}

// Sum over the kParts consecutive lanes of a column (an aligned group of 8
// or 16 lanes inside a 16-lane DPP row): quad permutes, then the half-row
// and row mirrors.  Every lane of the group ends with the same bits, since
// each step adds the same two values in either order.
template <int kParts>
__device__ __forceinline__ float part_sum(float v) {
  static_assert(kParts == 8 || kParts == 16, "parts per column");
  v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x141, 0xF>(v);  // row_half_mirror: sums over 8 lanes
  if constexpr (kParts == 16) v = dpp_add<0x140, 0xF>(v);  // row_mirror: sums over 16 lanes
  return v;
}

// Sum over the wave's 64 lanes: the 16-lane row sums, then row broadcasts 15
// and 31 carry rows 0-2 into row 3; lane 63 holds the total.
__device__ __forceinline__ float wave_sum(float v) {
  v = part_sum<16>(v);
  v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Raw buffer resource over `bytes` bytes at `base`: loads at offsets past
// the size return zeros, so the loads of tokens past the end (and of an
// absent v) need no branch.  A branch around a load makes the compiler wait
// for every load in flight at the next use of its registers, which would
// drain the prefetch ring at every token.
constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format
constexpr uint32_t kOutside = 0x80000000u;  // an offset past every resource used here
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const float* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, (int)bytes, kBufferFlags);
}
__device__ __forceinline__ float load1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ floatx4_t load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(floatx4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
typedef float floatx2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ floatx2_t load2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(floatx2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
// Stores go through buffer resources too: a store that must not happen
// (another lane of the column, a wave that does not own the value, an
// absent output) goes to a resource of size 0 and is dropped, so no store
// sits in a branch.
__device__ __forceinline__ void store1(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, 0);
}

// LDS writes made visible to the workgroup, then a barrier.  Unlike
// __syncthreads() this does not also wait for the loads in flight (the
// ring's prefetches), which would stall every barrier on them.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// kAhead = tokens of loads in flight (2 when 16 waves share the register
// file and a slot holds k and q: 2 x 16 + 2 values per lane).
// kO: the outputs o are asked for (else q is never read).
template <int kParts, int kCols, bool kNorms, bool kO, bool kVec>
__global__ __launch_bounds__(kParts * kCols) void gdn_recurrence_kernel(
    const float* __restrict__ x, int64_t ldx, int q_col, int k_col, int v_col, int g_col, int b_col, int T,
    int n_qk, int n_v, const float* __restrict__ s_in, float* __restrict__ s_out, float* __restrict__ o,
    int64_t ldo, float* __restrict__ norms, const int* __restrict__ snap_steps, int n_snaps,
    float* __restrict__ snaps) {
  constexpr int kRows = kD / kParts;     // rows of a column per lane
  constexpr int kThreads = kParts * kCols;
  constexpr int kGroups = kD / kCols;    // workgroups per value head
  constexpr int kAhead = kThreads > 256 && kO ? 2 : 4;
  constexpr int kChunk = 64;             // tokens per batch of per-token scalars
  static_assert(!kNorms || kGroups == 1, "the norm needs every column of the head in one workgroup");
  static_assert(kRows % 4 == 0, "rows per lane in 16-byte loads");
  static_assert(kThreads >= 256 && kChunk % kAhead == 0, "four waves compute the scalars of a chunk");
  const int h = blockIdx.x / kGroups;    // value head
  const int hk = h / (n_v / n_qk);       // its q / k head
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int part = tid % kParts;
  const int j = (blockIdx.x % kGroups) * kCols + tid / kParts;  // state column
  const int r0 = kRows * part;                                  // first state row of the lane
  const float rsd = 1.0f / sqrtf((float)kD);

  // per token of a chunk: 1 / |k|, 1 / (|q| sqrt(d)), alpha; two chunks
  __shared__ float scal[2][3][kChunk];
  // waves' shares of |S_t|_F^2 per token of a chunk, two chunks
  __shared__ float nsum[2][kNorms ? kThreads / 64 : 1][kNorms ? kChunk : 1];

  float S[kRows];
  {
    const float* si = s_in ? s_in + (int64_t)h * kD * kD : nullptr;
#pragma unroll
    for (int r = 0; r < kRows; ++r) S[r] = si ? si[(r0 + r) * kD + j] : 0.0f;
  }

  // this lane's rows of k and q, its value column and its head's gate columns
  const int64_t kc = k_col + (int64_t)hk * kD + r0, qc = q_col + (int64_t)hk * kD + r0;
  const int64_t vc = v_col >= 0 ? v_col + (int64_t)h * kD + j : -1;
  struct Tok {
    floatx4_t k[kRows / 4], q[kRows / 4];
    float v, b;
  };
  Tok ring[kAhead];
  const uint32_t row_bytes = (uint32_t)ldx * 4;
  auto fetch = [&](int t, Tok& c) {
    const bool live = t < T;
    const __amdgpu_buffer_rsrc_t r = rsrc(x + (int64_t)(live ? t : 0) * ldx, live ? row_bytes : 0);
#pragma unroll
    for (int i = 0; i < kRows / 4; ++i) {
      if constexpr (kVec) {
        c.k[i] = load4(r, (uint32_t)(kc + 4 * i) * 4);
        if constexpr (kO) c.q[i] = load4(r, (uint32_t)(qc + 4 * i) * 4);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          c.k[i][e] = load1(r, (uint32_t)(kc + 4 * i + e) * 4);
          if constexpr (kO) c.q[i][e] = load1(r, (uint32_t)(qc + 4 * i + e) * 4);
        }
      }
    }
    c.v = load1(r, vc >= 0 ? (uint32_t)vc * 4 : kOutside);
    c.b = load1(r, (uint32_t)(b_col + h) * 4);
  };

  // The scalars of a token (1 / |k|, 1 / (|q| sqrt(d)) and alpha = exp(g))
  // are the same for every lane of the head, so they are computed once per
  // chunk of 64 tokens instead of by every lane for every token.  The 128
  // vectors of a chunk (k and q of 64 tokens) are shared out over the waves,
  // kVecs each; a vector is read by the whole wave (two coalesced 256-byte
  // loads) and its squares summed with a DPP wave sum.  The loads of chunk
  // c + 1 are issued at the start of chunk c and held in registers (not in
  // the 16-wave form, which has no registers to spare: it loads them after
  // chunk c's tokens); its scalars are formed after chunk c's tokens, into
  // the other LDS buffer.
  constexpr int kWaves = kThreads / 64;
  constexpr bool kPrefetch = kWaves == 4;
  constexpr int kPerTok = kO ? 2 : 1;         // vectors per token: k (and q)
  constexpr int kVecs = kPerTok * kChunk / kWaves;  // vectors per wave per chunk
  float pre[kVecs][2];                        // two values of each of the wave's vectors per lane
  float pre_g = 0.0f;                         // wave 0: g of token c0 + lane
  auto chunk_load = [&](int c0) {
    const __amdgpu_buffer_rsrc_t r = rsrc(x + (int64_t)c0 * ldx, (int64_t)(min(T, c0 + kChunk) - c0) * row_bytes);
#pragma unroll
    for (int i = 0; i < kVecs; ++i) {
      const int vv = wave * kVecs + i;
      const uint32_t base = (uint32_t)(vv / kPerTok) * row_bytes + (uint32_t)((vv % kPerTok ? q_col : k_col) + hk * kD) * 4;
      if constexpr (kVec) {
        // 8-byte loads keep the loads in flight few: the wait for a ring
        // slot must be expressible in the wait counter (at most 63)
        const floatx2_t f = load2(r, base + (uint32_t)lane * 8);
        pre[i][0] = f[0];
        pre[i][1] = f[1];
      } else {
        pre[i][0] = load1(r, base + (uint32_t)lane * 4);
        pre[i][1] = load1(r, base + (uint32_t)(64 + lane) * 4);
      }
    }
    if (wave == 0) pre_g = load1(r, (uint32_t)lane * row_bytes + (uint32_t)(g_col + h) * 4);
  };
  auto chunk_scalars = [&](int buf) {
    float mine = 0.0f;  // lane i < kVecs: |vector wave * kVecs + i|^2
#pragma unroll
    for (int i = 0; i < kVecs; ++i) {
      const float ss = wave_sum(fmaf(pre[i][0], pre[i][0], pre[i][1] * pre[i][1]));
      mine = lane == i ? ss : mine;
    }
    if (lane < kVecs) {
      const int vv = wave * kVecs + lane;
      scal[buf][vv % kPerTok][vv / kPerTok] = (vv % kPerTok ? rsd : 1.0f) / fmaxf(sqrtf(mine), kNormEps);
    }
    if (wave == 0) scal[buf][2][lane] = expf(pre_g);
  };

  // One token of the recurrence, its values in ring slot a.  Inlined into
  // loops unrolled over the slots, so that a is a constant in each copy.
  auto token = [&](int t, int a, int c0, int buf, bool refill) {
    float kv[kRows], qv[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      kv[r] = ring[a].k[r / 4][r % 4];
      qv[r] = kO ? ring[a].q[r / 4][r % 4] : 0.0f;
    }
    const float v_t = ring[a].v, b_t = ring[a].b;
    const float rk = scal[buf][0][t - c0], alpha = scal[buf][2][t - c0];

    // u_j = S_{t-1}^T k (k not yet normalized: scaled by rk)
    float u0 = 0.0f, u1 = 0.0f;
#pragma unroll
    for (int r = 0; r < kRows; r += 2) {
      u0 = fmaf(S[r], kv[r], u0);
      u1 = fmaf(S[r + 1], kv[r + 1], u1);
    }
    const float u = part_sum<kParts>(u0 + u1) * rk;
    const float dk = b_t * (v_t - u) * rk;  // beta (v - u), times 1 / |k| for the raw k below

    // S_t = alpha S_{t-1} + khat (beta (v - u))^T, then o_j
    float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
    for (int r = 0; r < kRows; r += 2) {
      S[r] = fmaf(kv[r], dk, alpha * S[r]);
      S[r + 1] = fmaf(kv[r + 1], dk, alpha * S[r + 1]);
      if constexpr (kO) {
        o0 = fmaf(S[r], qv[r], o0);
        o1 = fmaf(S[r + 1], qv[r + 1], o1);
      }
    }
    if constexpr (kO) {
      const float ov = part_sum<kParts>(o0 + o1) * scal[buf][1][t - c0];
      store1(rsrc(o + (int64_t)t * ldo, (int64_t)(h + 1) * kD * 4), part == 0 ? (uint32_t)(h * kD + j) * 4 : kOutside,
             ov);
    }

    // keep the refill right here: left alone, the scheduler sinks the
    // refills to the end of the loop body, and the next token then
    // waits for nearly every load in flight
    __builtin_amdgcn_sched_barrier(0);
    if (refill) fetch(t + kAhead, ring[a]);
    __builtin_amdgcn_sched_barrier(0);

    if constexpr (kNorms) {
      // |S_t|_F^2: each wave's share goes to LDS; the shares of a chunk are
      // added after the chunk's barrier (no barrier per token)
      float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
      for (int r = 0; r < kRows; r += 2) {
        s0 = fmaf(S[r], S[r], s0);
        s1 = fmaf(S[r + 1], S[r + 1], s1);
      }
      const float ws = wave_sum(s0 + s1);
      if (lane == 0) nsum[buf][wave][t - c0] = ws;
    }
  };

  // Snapshots split the tokens into segments, each run from a fresh ring
  // and chunk sequence, with the state written out between them: the
  // token loop itself has no branch that stores, which would make the
  // compiler wait for every load in flight at the next token.
  int sb = 0;
  for (int si = 0; sb < T || si < n_snaps; ++si) {
    int se = T;  // this segment: tokens sb .. se - 1
    bool snap = false;
    if (si < n_snaps) {
      const int st = snap_steps[si];
      snap = st >= sb && st < T;  // steps out of order are skipped
      se = snap ? st + 1 : sb;
    } else if (sb >= T) {
      break;
    }
#pragma unroll
    for (int a = 0; a < kAhead; ++a) fetch(sb + a, ring[a]);
    if (sb < se) {
      chunk_load(sb);
      chunk_scalars(0);
      lds_barrier();
    }
    for (int c0 = sb; c0 < se; c0 += kChunk) {
      const int buf = ((c0 - sb) / kChunk) & 1;
      if (kPrefetch && c0 + kChunk < se) chunk_load(c0 + kChunk);
      const int c1 = min(c0 + kChunk, se);
      // The loop is unrolled by kAhead so that token t always finds its
      // values in slot (t - sb) % kAhead, refilled in place with token
      // t + kAhead: a loaded register is never moved (a move would wait for
      // its load).  Only whole groups of kAhead tokens run in the loop; a
      // branch out of its body (at the last tokens) would make the compiler
      // wait for every load in flight at the top of the next group.
      int t0 = c0;
      for (; t0 + kAhead <= c1; t0 += kAhead) {
#pragma unroll
        for (int a = 0; a < kAhead; ++a) token(t0 + a, a, c0, buf, true);
      }
      // the segment's last tokens: no refill (the next segment starts a new
      // ring), so no load sits in a branch
#pragma unroll
      for (int a = 0; a + 1 < kAhead; ++a)
        if (t0 + a < c1) token(t0 + a, a, c0, buf, false);
      // the next chunk's scalars go to the other buffer; after the barrier
      // every wave is also done with this chunk's, which chunk c + 2 rewrites
      if (c0 + kChunk < se) {
        if (!kPrefetch) chunk_load(c0 + kChunk);
        chunk_scalars(buf ^ 1);
      }
      lds_barrier();
      if constexpr (kNorms) {
        // |S_t|_F^2 of the chunk's tokens, lane l of wave 0 for token c0 + l
        // (waves added in a fixed order); the buffer is rewritten two chunks
        // later, after another barrier
        if (wave == 0) {
          float ns = 0.0f;
#pragma unroll
          for (int w = 0; w < kThreads / 64; ++w) ns += nsum[buf][w][lane];
          store1(rsrc(norms + (int64_t)c0 * n_v, norms ? (int64_t)(c1 - c0) * n_v * 4 : 0),
                 (uint32_t)(lane * n_v + h) * 4, ns);
        }
      }
    }
    if (snap) {
      float* dst = snaps + ((int64_t)si * n_v + h) * kD * kD;
#pragma unroll
      for (int r = 0; r < kRows; ++r) dst[(r0 + r) * kD + j] = S[r];
    }
    sb = se;
  }
  if (s_out) {
    float* so = s_out + (int64_t)h * kD * kD;
#pragma unroll
    for (int r = 0; r < kRows; ++r) so[(r0 + r) * kD + j] = S[r];
  }
}

template <int kParts, int kCols, bool kNorms, bool kO>
hipError_t launch_variant(bool vec, const float* x, int64_t ldx, int64_t q_col, int64_t k_col, int64_t v_col,
                          int64_t g_col, int64_t b_col, int64_t T, int n_qk, int n_v, const float* s_in,
                          float* s_out, float* o, int64_t ldo, float* norms, const int* snap_steps, int n_snaps,
                          float* snaps, hipStream_t stream) {
  const dim3 grid((unsigned)(n_v * (kD / kCols))), block(kParts * kCols);
  if (vec)
    gdn_recurrence_kernel<kParts, kCols, kNorms, kO, true><<<grid, block, 0, stream>>>(
        x, ldx, (int)q_col, (int)k_col, (int)v_col, (int)g_col, (int)b_col, (int)T, n_qk, n_v, s_in, s_out, o,
        ldo, norms, snap_steps, n_snaps, snaps);
  else
    gdn_recurrence_kernel<kParts, kCols, kNorms, kO, false><<<grid, block, 0, stream>>>(
        x, ldx, (int)q_col, (int)k_col, (int)v_col, (int)g_col, (int)b_col, (int)T, n_qk, n_v, s_in, s_out, o,
        ldo, norms, snap_steps, n_snaps, snaps);
  return hipGetLastError();
}

// S_0 = the start state (zeros without one), element by element; in and
// out may be the same buffer.
__global__ void gdn_start_state_kernel(const float* in, float* out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = in ? in[i] : 0.0f;
}

}  // namespace

hipError_t launch_gdn_start_state(const float* s_in, float* s_out, int n_v, hipStream_t stream) {
  const int64_t n = (int64_t)n_v * kD * kD;
  gdn_start_state_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(s_in, s_out, n);
  return hipGetLastError();
}

hipError_t launch_gdn_recurrence(const float* x, int64_t ldx, int64_t q_col, int64_t k_col, int64_t v_col,
                                 int64_t g_col, int64_t b_col, int64_t T, int n_qk, int n_v, const float* s_in,
                                 float* s_out, float* o, int64_t ldo, float* norms, const int* snap_steps,
                                 int n_snaps, float* snaps, hipStream_t stream) {
  // 16-byte loads of k and q when every row's k and q start 16-byte aligned
  const bool vec = (uintptr_t)x % 16 == 0 && ldx % 4 == 0 && q_col % 4 == 0 && k_col % 4 == 0;
#define NVFP4_GDN(P, C, N, O)                                                                                 \
  return launch_variant<P, C, N, O>(vec, x, ldx, q_col, k_col, v_col, g_col, b_col, T, n_qk, n_v, s_in, s_out, o, \
                                    ldo, norms, snap_steps, n_snaps, snaps, stream)
  if (norms) {
    if (o) NVFP4_GDN(8, kD, true, true);
    NVFP4_GDN(8, kD, true, false);
  }
  if (o) NVFP4_GDN(16, 16, false, true);
  NVFP4_GDN(16, 16, false, false);
#undef NVFP4_GDN
}

}  // namespace nvfp4
