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
// head h reads q/k head h * n_qk / n_v.
//
// One workgroup of 1024 threads (16 waves, four per SIMD) per value head,
// d_k = d_v = 128.  Thread t owns column j = t % 128 of S and its rows
// 16 (t / 128) .. + 15, in registers.  Per token:
//   * k and q (2 x 128 values) were staged in LDS during the previous token,
//     one value per thread of waves 0-3, with their squared norms reduced
//     per wave;
//   * u_j: each thread sums its 16 rows, the eight parts meet in LDS (barrier);
//   * the update of the thread's 16 state values, then its part of o_j;
//   * the next token's k / q go to the other LDS buffer, and the parts of
//     o_j meet (barrier).
// (Two parts of 64 rows on 256 threads took 1.75 us per token, four parts
// 1.39 us, eight 1.32 us.)
// Loads of the projection rows run 4 tokens ahead in registers (a ring of
// slots indexed at compile time), so the sequential loop does not wait on
// memory.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

constexpr int kD = 128;       // head dimension (d_k = d_v)
constexpr int kSplit = 8;     // threads per state column: each holds kD / kSplit rows
constexpr int kRows = kD / kSplit;
constexpr int kThreads = kD * kSplit;
constexpr int kAhead = 4;     // tokens of loads in flight
constexpr float kNormEps = 1e-6f;

// Sum over the wave's 64 lanes with DPP (no LDS round trips): quad
// permutes, half-row and row mirrors give every lane its 16-lane row's sum,
// then row broadcasts 15 and 31 carry rows 0-2 into row 3; lane 63 holds the
// total, returned to every lane.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_add<0x140, 0xF>(v);  // row_mirror
  v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__global__ __launch_bounds__(kThreads) void gdn_recurrence_kernel(
    const float* __restrict__ x, int64_t ldx, int q_col, int k_col, int v_col, int g_col, int b_col, int T,
    int n_qk, int n_v, const float* __restrict__ s_in, float* __restrict__ s_out, float* __restrict__ o,
    int64_t ldo, float* __restrict__ norms, const int* __restrict__ snap_steps, int n_snaps,
    float* __restrict__ snaps) {
  const int h = blockIdx.x;              // value head
  const int hk = h / (n_v / n_qk);       // its q / k head
  const int tid = threadIdx.x, j = tid & (kD - 1), hf = tid >> 7;  // column, row part
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;

  __shared__ __attribute__((aligned(16))) float kq[2][2 * kD];  // [buffer][k 0..127 | q 128..255]
  __shared__ float nrm[2][4];                                   // [buffer][wave]: k (waves 0, 1), q (2, 3)
  __shared__ float part[2][kSplit][kD];                         // [u | o][row part][column]
  __shared__ float nsum[kThreads / 64];

  float S[kRows];
  {
    const float* si = s_in ? s_in + (int64_t)h * kD * kD : nullptr;
#pragma unroll
    for (int r = 0; r < kRows; ++r) S[r] = si ? si[(kRows * hf + r) * kD + j] : 0.0f;
  }

  // this thread's staged element (k for tid < 128, q for tid < 256; the
  // other threads stage nothing), its value column and its head's gate
  // columns
  const bool stager = tid < 2 * kD;
  const int64_t sc = (tid < kD ? k_col : q_col) + (int64_t)hk * kD + j;
  const int64_t vc = v_col >= 0 ? v_col + (int64_t)h * kD + j : -1;
  float p_s[kAhead], p_v[kAhead], p_g[kAhead], p_b[kAhead];
  auto fetch = [&](int t, float& s, float& v, float& g, float& b) {
    if (t < T) {
      const float* row = x + (int64_t)t * ldx;
      s = stager ? row[sc] : 0.0f;
      v = vc >= 0 ? row[vc] : 0.0f;
      g = row[g_col + h];
      b = row[b_col + h];
    } else {
      s = v = g = b = 0.0f;
    }
  };
#pragma unroll
  for (int a = 0; a < kAhead; ++a) fetch(a, p_s[a], p_v[a], p_g[a], p_b[a]);

  auto stage = [&](float s, int buf) {
    if (stager) {  // waves 0-3 (uniform per wave)
      kq[buf][tid] = s;
      const float sq = wave_sum(s * s);
      if (lane == 0) nrm[buf][wave] = sq;
    }
  };
  stage(p_s[0], 0);
  __syncthreads();

  int snap_i = 0;
  int next_snap = (snap_steps && n_snaps > 0) ? snap_steps[0] : -1;
  const float rsd = 1.0f / sqrtf((float)kD);

  // The loop is unrolled by kAhead so that token t always finds its values
  // in slot t % kAhead, refilled in place with token t + kAhead: a loaded
  // register is never moved (a move would wait for its load).
  for (int t0 = 0; t0 < T; t0 += kAhead) {
#pragma unroll
    for (int a = 0; a < kAhead; ++a) {
      const int t = t0 + a;
      if (t >= T) break;
      const int buf = t & 1;
      const float v_t = p_v[a], g_t = p_g[a], b_t = p_b[a];

      const float* kv = &kq[buf][kRows * hf];
      const float* qv = &kq[buf][kD + kRows * hf];
      const float rk = 1.0f / fmaxf(sqrtf(nrm[buf][0] + nrm[buf][1]), kNormEps);
      const float rq = rsd / fmaxf(sqrtf(nrm[buf][2] + nrm[buf][3]), kNormEps);

      // u_j = S_{t-1}^T k (k not yet normalized: scaled by rk below); eight
      // independent partial sums, so the sum is not one long chain of FMAs
      float acc[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
#pragma unroll
      for (int r = 0; r < kRows; ++r) acc[r & 7] = fmaf(S[r], kv[r], acc[r & 7]);
      part[0][hf][j] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
      __syncthreads();
      float usum = 0.0f;
#pragma unroll
      for (int p = 0; p < kSplit; ++p) usum += part[0][p][j];
      const float u = usum * rk;
      const float alpha = expf(g_t);
      const float dk = b_t * (v_t - u) * rk;  // beta (v - u), times 1 / |k| for the raw k below

      // S_t = alpha S_{t-1} + khat (beta (v - u))^T, then o's partial
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        S[r] = fmaf(kv[r], dk, alpha * S[r]);
        acc[r & 7] = fmaf(S[r], qv[r], acc[r & 7]);
      }
      part[1][hf][j] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
      if (norms) {
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
#pragma unroll
        for (int r = 0; r < kRows; ++r) acc[r & 7] = fmaf(S[r], S[r], acc[r & 7]);
        const float ps = wave_sum(((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7])));
        if (lane == 0) nsum[wave] = ps;
      }
      stage(p_s[(a + 1) % kAhead], buf ^ 1);  // token t + 1
      fetch(t + kAhead, p_s[a], p_v[a], p_g[a], p_b[a]);
      __syncthreads();

      if (o && hf == 0) {
        float osum = 0.0f;
#pragma unroll
        for (int p = 0; p < kSplit; ++p) osum += part[1][p][j];
        o[(int64_t)t * ldo + (int64_t)h * kD + j] = osum * rq;
      }
      if (norms && tid == 0) {
        float ns = 0.0f;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) ns += nsum[w];
        norms[(int64_t)t * n_v + h] = ns;
      }
      if (t == next_snap) {
        float* dst = snaps + ((int64_t)snap_i * n_v + h) * kD * kD;
#pragma unroll
        for (int r = 0; r < kRows; ++r) dst[(kRows * hf + r) * kD + j] = S[r];
        ++snap_i;
        next_snap = snap_i < n_snaps ? snap_steps[snap_i] : -1;
      }
    }
  }
  if (s_out) {
    float* so = s_out + (int64_t)h * kD * kD;
#pragma unroll
    for (int r = 0; r < kRows; ++r) so[(kRows * hf + r) * kD + j] = S[r];
  }
}

}  // namespace

hipError_t launch_gdn_recurrence(const float* x, int64_t ldx, int64_t q_col, int64_t k_col, int64_t v_col,
                                 int64_t g_col, int64_t b_col, int64_t T, int n_qk, int n_v, const float* s_in,
                                 float* s_out, float* o, int64_t ldo, float* norms, const int* snap_steps,
                                 int n_snaps, float* snaps, hipStream_t stream) {
  gdn_recurrence_kernel<<<dim3((unsigned)n_v), dim3(kThreads), 0, stream>>>(
      x, ldx, (int)q_col, (int)k_col, (int)v_col, (int)g_col, (int)b_col, (int)T, n_qk, n_v, s_in, s_out, o, ldo,
      norms, snap_steps, n_snaps, snaps);
  return hipGetLastError();
}

}  // namespace nvfp4
