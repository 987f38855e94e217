// C ABI of the NVFP4 library: argument validation, then dispatch to the
// kernel launchers.  Every check runs before the first HIP call, so a bad
// argument never enqueues work (and the checks run on machines without a GPU).
#include "../../include/nvfp4.h"

#include <hip/hip_runtime.h>

#include <climits>

#include "nvfp4_internal.h"

namespace {

thread_local int32_t g_last_hip_error = 0;

nvfp4_status_t hip_status(hipError_t e) {
  if (e == hipSuccess) return NVFP4_OK;
  g_last_hip_error = (int32_t)e;
  return NVFP4_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Checks shared by nvfp4_gemm and nvfp4_gemm_segmented (the caller has
// filled the column scale table), then the launch.
nvfp4_status_t gemm_checked(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
                            const uint8_t* w_codes, const uint8_t* w_scales, const nvfp4::ColScales& cs,
                            int64_t M, int64_t N, int64_t K, void* y, int32_t out_dtype, int64_t ldy,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (out_dtype != NVFP4_OUT_F32 && out_dtype != NVFP4_OUT_BF16) return NVFP4_ERR_DTYPE;
  if (M < 0 || N <= 0 || K <= 0 || K % 16 != 0 || ldy < N) return NVFP4_ERR_SHAPE;
  if (M > INT_MAX || N > INT_MAX || K > INT_MAX) return NVFP4_ERR_SHAPE;
  if (M == 0) return NVFP4_OK;
  if (!a_codes || !a_scales || !a_gs || !w_codes || !w_scales || !cs.gs || !y) return NVFP4_ERR_NULL;
  if (!aligned(a_gs, 4) || !aligned(cs.gs, 4) || !aligned(y, out_dtype == NVFP4_OUT_BF16 ? 2 : 4))
    return NVFP4_ERR_ALIGN;
  const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
  if (tiles > (int64_t)INT_MAX) return NVFP4_ERR_SHAPE;
  const size_t need = nvfp4::gemm_split_workspace_bytes(M, N, K);
  if (workspace_bytes < need) return NVFP4_ERR_WORKSPACE;
  if (need > 0 && !workspace) return NVFP4_ERR_NULL;
  if (need > 0 && !aligned(workspace, 16)) return NVFP4_ERR_ALIGN;
  return hip_status(nvfp4::launch_gemm(a_codes, a_scales, a_gs, w_codes, w_scales, cs, M, N, K, y,
                                       out_dtype == NVFP4_OUT_BF16, ldy, (hipStream_t)stream,
                                       need > 0 ? workspace : nullptr, need));
}


// Argument checks of nvfp4_quantize_gemm and its allocation-free variant
// (everything but the workspace), before any HIP call.
nvfp4_status_t quantize_gemm_checks(const void* x, int32_t in_dtype, int64_t ldx, const float* a_gs,
                                    const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gs, int64_t M,
                                    int64_t N, int64_t K, void* y, int32_t out_dtype, int64_t ldy) {
  if (in_dtype != NVFP4_IN_F32 && in_dtype != NVFP4_IN_BF16) return NVFP4_ERR_DTYPE;
  if (out_dtype != NVFP4_OUT_F32 && out_dtype != NVFP4_OUT_BF16) return NVFP4_ERR_DTYPE;
  if (M < 0 || N <= 0 || K <= 0 || K % 16 != 0 || ldx < K || ldy < N) return NVFP4_ERR_SHAPE;
  if (M > INT_MAX || N > INT_MAX || K > INT_MAX || M > INT64_MAX / ldx / 4) return NVFP4_ERR_SHAPE;
  if (M == 0) return NVFP4_OK;
  if (!x || !a_gs || !w_codes || !w_scales || !w_gs || !y) return NVFP4_ERR_NULL;
  const int64_t esize = in_dtype == NVFP4_IN_BF16 ? 2 : 4;
  if (!aligned(x, 16) || (ldx * esize) % 16 != 0 || !aligned(a_gs, 4) || !aligned(w_gs, 4) ||
      !aligned(y, out_dtype == NVFP4_OUT_BF16 ? 2 : 4))
    return NVFP4_ERR_ALIGN;
  if ((M * (K / 16) + 255) / 256 > (int64_t)INT_MAX) return NVFP4_ERR_SHAPE;
  if (((M + 127) / 128) * ((N + 127) / 128) > (int64_t)INT_MAX) return NVFP4_ERR_SHAPE;
  if (nvfp4_quantize_gemm_workspace_size(M, N, K, in_dtype, out_dtype) == 0 &&
      (!aligned(w_codes, 16) || !aligned(w_scales, 8)))
    return NVFP4_ERR_ALIGN;  // the one-kernel form reads W with 16- and 4-byte loads
  return NVFP4_OK;
}

// The launches of a checked quantize + GEMM: one kernel when `need` is 0,
// else the quantize kernel into ws (codes, then scales 256-byte aligned)
// and the GEMM from there.
nvfp4_status_t quantize_gemm_launch(const void* x, int32_t in_dtype, int64_t ldx, const float* a_gs,
                                    const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gs, int64_t M,
                                    int64_t N, int64_t K, void* y, int32_t out_dtype, int64_t ldy, uint8_t* ws,
                                    size_t need, void* stream) {
  nvfp4::ColScales cs{};
  cs.gs = w_gs;
  cs.n = 1;
  cs.end[0] = (int)N;
  const bool in_bf16 = in_dtype == NVFP4_IN_BF16, out_bf16 = out_dtype == NVFP4_OUT_BF16;
  if (need == 0)  // one kernel: the decode GEMM quantizes the activations itself
    return hip_status(nvfp4::launch_quantize_gemm_fused(x, in_bf16, ldx, a_gs, w_codes, w_scales, cs, M, N, K, y,
                                                        out_bf16, ldy, (hipStream_t)stream));
  uint8_t* codes = ws;
  uint8_t* scales = codes + (M * (K / 2) + 255) / 256 * 256;
  const nvfp4_status_t st = hip_status(nvfp4::launch_quantize(x, in_bf16, M, K, ldx, codes, scales,
                                                              const_cast<float*>(a_gs), false, (hipStream_t)stream));
  if (st != NVFP4_OK) return st;
  return hip_status(nvfp4::launch_gemm(codes, scales, a_gs, w_codes, w_scales, cs, M, N, K, y, out_bf16, ldy,
                                       (hipStream_t)stream));
}

}  // namespace

extern "C" {

nvfp4_status_t nvfp4_quantize(const void* x, int32_t in_dtype, int64_t rows, int64_t cols,
                              int64_t ldx, uint8_t* codes, uint8_t* scales,
                              float* global_scale, int32_t mode, void* stream) {
  try {
    if (in_dtype != NVFP4_IN_F32 && in_dtype != NVFP4_IN_BF16) return NVFP4_ERR_DTYPE;
    if (mode != NVFP4_SCALE_GIVEN && mode != NVFP4_SCALE_FROM_AMAX) return NVFP4_ERR_MODE;
    if (rows < 0 || cols <= 0 || cols % 16 != 0 || ldx < cols) return NVFP4_ERR_SHAPE;
    if (rows > INT64_MAX / (ldx > 0 ? ldx : 1) / 4) return NVFP4_ERR_SHAPE;
    if (rows == 0) {  // nothing to encode; FROM_AMAX still writes g (1.0: no values, amax 0)
      if (mode == NVFP4_SCALE_GIVEN) return NVFP4_OK;
      if (!global_scale) return NVFP4_ERR_NULL;
      if (!aligned(global_scale, 4)) return NVFP4_ERR_ALIGN;
      return hip_status(nvfp4::launch_quantize(nullptr, in_dtype == NVFP4_IN_BF16, 0, cols, ldx, nullptr, nullptr,
                                               global_scale, true, (hipStream_t)stream));
    }
    if (!x || !codes || !scales || !global_scale) return NVFP4_ERR_NULL;
    const int64_t esize = in_dtype == NVFP4_IN_BF16 ? 2 : 4;
    if (!aligned(x, 16) || (ldx * esize) % 16 != 0 || !aligned(codes, 8) || !aligned(global_scale, 4))
      return NVFP4_ERR_ALIGN;
    if ((rows * (cols / 16) + 255) / 256 > (int64_t)INT_MAX) return NVFP4_ERR_SHAPE;
    return hip_status(nvfp4::launch_quantize(x, in_dtype == NVFP4_IN_BF16, rows, cols, ldx, codes,
                                             scales, global_scale, mode == NVFP4_SCALE_FROM_AMAX,
                                             (hipStream_t)stream));
  } catch (...) {
    return NVFP4_ERR_HIP;
  }
}

size_t nvfp4_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int32_t out_dtype) {
  (void)out_dtype;
  if (M <= 0 || N <= 0 || K <= 0 || M > INT_MAX || N > INT_MAX || K > INT_MAX) return 0;
  return nvfp4::gemm_split_workspace_bytes(M, N, K);
}

nvfp4_status_t nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
                          const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gs,
                          int64_t M, int64_t N, int64_t K, void* y, int32_t out_dtype,
                          int64_t ldy, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    nvfp4::ColScales cs{};
    cs.gs = w_gs;
    cs.n = 1;
    cs.end[0] = (N > 0 && N <= INT_MAX) ? (int)N : 0;  // out-of-range N fails the shape check
    return gemm_checked(a_codes, a_scales, a_gs, w_codes, w_scales, cs, M, N, K, y, out_dtype, ldy,
                        workspace, workspace_bytes, stream);
  } catch (...) {
    return NVFP4_ERR_HIP;
  }
}

nvfp4_status_t nvfp4_gemm_segmented(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
                                    const uint8_t* w_codes, const uint8_t* w_scales,
                                    const float* module_gs, const int64_t* module_rows, int32_t n_modules,
                                    int64_t M, int64_t K, void* y, int32_t out_dtype, int64_t ldy,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  try {
    if (!module_rows) return NVFP4_ERR_NULL;
    if (n_modules < 1 || n_modules > nvfp4::kMaxModules) return NVFP4_ERR_SHAPE;
    nvfp4::ColScales cs{};
    cs.gs = module_gs;
    cs.n = n_modules;
    int64_t N = 0;
    for (int32_t i = 0; i < n_modules; ++i) {
      if (module_rows[i] < 0 || module_rows[i] > (int64_t)INT_MAX - N) return NVFP4_ERR_SHAPE;
      N += module_rows[i];
      cs.end[i] = (int)N;
    }
    return gemm_checked(a_codes, a_scales, a_gs, w_codes, w_scales, cs, M, N, K, y, out_dtype, ldy,
                        workspace, workspace_bytes, stream);
  } catch (...) {
    return NVFP4_ERR_HIP;
  }
}

nvfp4_status_t nvfp4_gemm_segmented_gates(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
                                          const uint8_t* w_codes, const uint8_t* w_scales,
                                          const float* module_gs, const int64_t* module_rows, int32_t n_modules,
                                          int32_t decay_module, const float* a_log, const float* dt_bias,
                                          int32_t write_module, int64_t M, int64_t K, void* y, int32_t out_dtype,
                                          int64_t ldy, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    if (!module_rows) return NVFP4_ERR_NULL;
    if (n_modules < 1 || n_modules > nvfp4::kMaxModules) return NVFP4_ERR_SHAPE;
    if (decay_module < -1 || decay_module >= n_modules || write_module < -1 || write_module >= n_modules)
      return NVFP4_ERR_SHAPE;
    if (decay_module >= 0 && decay_module == write_module) return NVFP4_ERR_SHAPE;
    if (decay_module >= 0) {
      if (!a_log || !dt_bias) return NVFP4_ERR_NULL;
      if (!aligned(a_log, 4) || !aligned(dt_bias, 4)) return NVFP4_ERR_ALIGN;
    }
    nvfp4::ColScales cs{};
    cs.gs = module_gs;
    cs.n = n_modules;
    int64_t N = 0;
    for (int32_t i = 0; i < n_modules; ++i) {
      if (module_rows[i] < 0 || module_rows[i] > (int64_t)INT_MAX - N) return NVFP4_ERR_SHAPE;
      if (i == decay_module) cs.decay_lo = (int)N, cs.decay_hi = (int)(N + module_rows[i]);
      if (i == write_module) cs.write_lo = (int)N, cs.write_hi = (int)(N + module_rows[i]);
      N += module_rows[i];
      cs.end[i] = (int)N;
    }
    cs.a_log = a_log;
    cs.dt_bias = dt_bias;
    return gemm_checked(a_codes, a_scales, a_gs, w_codes, w_scales, cs, M, N, K, y, out_dtype, ldy,
                        workspace, workspace_bytes, stream);
  } catch (...) {
    return NVFP4_ERR_HIP;
  }
}

nvfp4_status_t nvfp4_gdn_recurrence(const float* x, int64_t ldx, int64_t q_col, int64_t k_col, int64_t v_col,
                                    int64_t g_col, int64_t beta_col, int64_t T, int32_t n_qk_heads,
                                    int32_t n_v_heads, const float* state_in, float* state_out, float* o,
                                    int64_t ldo, float* state_norms, const int32_t* snap_steps, int32_t n_snaps,
                                    float* snaps, void* stream) {
  try {
    constexpr int64_t kD = 128;
    // rows of fewer than 2^23 values: 64 rows of the chunk loads stay below 2^31 bytes
    if (T < 0 || T > INT_MAX || ldx <= 0 || ldx >= ((int64_t)1 << 23)) return NVFP4_ERR_SHAPE;
    if (n_qk_heads < 1 || n_v_heads < 1 || n_v_heads > 65535 || n_v_heads % n_qk_heads != 0) return NVFP4_ERR_SHAPE;
    if (q_col < 0 || q_col + n_qk_heads * kD > ldx || k_col < 0 || k_col + n_qk_heads * kD > ldx)
      return NVFP4_ERR_SHAPE;
    if (v_col < -1 || (v_col >= 0 && v_col + n_v_heads * kD > ldx)) return NVFP4_ERR_SHAPE;
    if (g_col < 0 || g_col + n_v_heads > ldx || beta_col < 0 || beta_col + n_v_heads > ldx) return NVFP4_ERR_SHAPE;
    if (o && ldo < n_v_heads * kD) return NVFP4_ERR_SHAPE;
    if (n_snaps < 0) return NVFP4_ERR_SHAPE;
    if (T == 0) {  // S_0 is the start state; nothing else has a row to write
      if (!state_out) return NVFP4_OK;
      if (!aligned(state_out, 4) || (state_in && !aligned(state_in, 4))) return NVFP4_ERR_ALIGN;
      return hip_status(nvfp4::launch_gdn_start_state(state_in, state_out, n_v_heads, (hipStream_t)stream));
    }
    if (!x || (n_snaps > 0 && (!snap_steps || !snaps))) return NVFP4_ERR_NULL;
    for (const void* p : {(const void*)x, (const void*)state_in, (const void*)state_out, (const void*)o,
                          (const void*)state_norms, (const void*)snap_steps, (const void*)snaps})
      if (p && !aligned(p, 4)) return NVFP4_ERR_ALIGN;
    return hip_status(nvfp4::launch_gdn_recurrence(x, ldx, q_col, k_col, v_col, g_col, beta_col, T, n_qk_heads,
                                                   n_v_heads, state_in, state_out, o, ldo, state_norms,
                                                   snap_steps, n_snaps > 0 ? n_snaps : 0, snaps,
                                                   (hipStream_t)stream));
  } catch (...) {
    return NVFP4_ERR_HIP;
  }
}

nvfp4_status_t nvfp4_gemm_swiglu_quantize(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
                                          const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gs,
                                          int64_t M, int64_t F, int64_t K, const float* h_gs, uint8_t* h_codes,
                                          uint8_t* h_scales, float* h, int64_t ldh, void* stream) {
  try {
    if (M < 0 || F <= 0 || K <= 0 || K % 128 != 0 || F % 64 != 0) return NVFP4_ERR_SHAPE;
    if (M > INT_MAX || F > INT_MAX / 2 || K > INT_MAX) return NVFP4_ERR_SHAPE;
    if (h && ldh < F) return NVFP4_ERR_SHAPE;
    // 32-bit buffer offsets of the streaming kernel
    if (M * (K / 2) >= ((int64_t)1 << 31) || 2 * F * (K / 2) >= ((int64_t)1 << 31)) return NVFP4_ERR_SHAPE;
    if (M == 0) return NVFP4_OK;
    if (!a_codes || !a_scales || !a_gs || !w_codes || !w_scales || !w_gs || !h_gs || !h_codes || !h_scales)
      return NVFP4_ERR_NULL;
    if (!aligned(a_codes, 16) || !aligned(w_codes, 16) || !aligned(a_scales, 8) || !aligned(w_scales, 8) ||
        !aligned(a_gs, 4) || !aligned(w_gs, 4) || !aligned(h_gs, 4) || !aligned(h_codes, 8) ||
        (h && (!aligned(h, 16) || ldh % 4 != 0)))
      return NVFP4_ERR_ALIGN;
    if (((M + 255) / 256) * ((2 * F + 255) / 256) > (int64_t)INT_MAX) return NVFP4_ERR_SHAPE;
    nvfp4::SwigluOut out{h_gs, h_codes, h_scales, h, ldh, (int)F};
    return hip_status(nvfp4::launch_gemm_swiglu_quantize(a_codes, a_scales, a_gs, w_codes, w_scales, w_gs, M, F, K,
                                                         out, (hipStream_t)stream));
  } catch (...) {
    return NVFP4_ERR_HIP;
  }
}

size_t nvfp4_quantize_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int32_t in_dtype, int32_t out_dtype) {
  (void)out_dtype;
  if (M <= 0 || N <= 0 || K <= 0 || K % 16 != 0 || M > INT_MAX || K > INT_MAX) return 0;
  if (nvfp4::quantize_gemm_fused_fits(M, N, K, in_dtype == NVFP4_IN_BF16)) return 0;
  const int64_t code_bytes = (M * (K / 2) + 255) / 256 * 256;  // scales start 256-byte aligned
  return (size_t)(code_bytes + M * (K / 16));
}

nvfp4_status_t nvfp4_quantize_gemm(const void* x, int32_t in_dtype, int64_t ldx, const float* a_gs,
                                   const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gs,
                                   int64_t M, int64_t N, int64_t K, void* y, int32_t out_dtype, int64_t ldy,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  try {
    const nvfp4_status_t st = quantize_gemm_checks(x, in_dtype, ldx, a_gs, w_codes, w_scales, w_gs, M, N, K, y,
                                                   out_dtype, ldy);
    if (st != NVFP4_OK || M == 0) return st;
    const size_t need = nvfp4_quantize_gemm_workspace_size(M, N, K, in_dtype, out_dtype);
    if (workspace_bytes < need) return NVFP4_ERR_WORKSPACE;
    if (need > 0 && !workspace) return NVFP4_ERR_NULL;
    if (need > 0 && !aligned(workspace, 16)) return NVFP4_ERR_ALIGN;
    return quantize_gemm_launch(x, in_dtype, ldx, a_gs, w_codes, w_scales, w_gs, M, N, K, y, out_dtype, ldy,
                                static_cast<uint8_t*>(workspace), need, stream);
  } catch (...) {
    return NVFP4_ERR_HIP;
  }
}

nvfp4_status_t nvfp4_quantize_gemm_no_alloc(const void* x, int32_t in_dtype, int64_t ldx, const float* a_gs,
                                            const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gs,
                                            int64_t M, int64_t N, int64_t K, void* y, int32_t out_dtype,
                                            int64_t ldy, void* stream) {
  try {
    const nvfp4_status_t st = quantize_gemm_checks(x, in_dtype, ldx, a_gs, w_codes, w_scales, w_gs, M, N, K, y,
                                                   out_dtype, ldy);
    if (st != NVFP4_OK || M == 0) return st;
    const size_t need = nvfp4_quantize_gemm_workspace_size(M, N, K, in_dtype, out_dtype);
    if (need > nvfp4::kNoAllocScratchBytes) return NVFP4_ERR_TOO_LARGE;
    void* scratch = nullptr;
    if (need > 0) {
      const hipError_t e = nvfp4::no_alloc_scratch(&scratch);
      if (e != hipSuccess) return hip_status(e);
    }
    return quantize_gemm_launch(x, in_dtype, ldx, a_gs, w_codes, w_scales, w_gs, M, N, K, y, out_dtype, ldy,
                                static_cast<uint8_t*>(scratch), need, stream);
  } catch (...) {
    return NVFP4_ERR_HIP;
  }
}

size_t nvfp4_quantize_gemm_no_alloc_max_bytes(void) { return nvfp4::kNoAllocScratchBytes; }

nvfp4_status_t nvfp4_harmonize_fused_scales(uint8_t* scales, const float* module_gs,
                                            const int64_t* module_rows, int32_t n_modules,
                                            int64_t K, float* shared_gs, uint32_t* counters,
                                            void* stream) {
  try {
    if (!scales || !module_gs || !module_rows || !shared_gs) return NVFP4_ERR_NULL;
    if (n_modules < 1 || n_modules > nvfp4::kMaxModules) return NVFP4_ERR_SHAPE;
    if (K <= 0 || K % 16 != 0) return NVFP4_ERR_SHAPE;
    int64_t total = 0;
    for (int32_t i = 0; i < n_modules; ++i) {
      if (module_rows[i] < 0 || module_rows[i] > INT64_MAX / 2 - total) return NVFP4_ERR_SHAPE;
      total += module_rows[i];
    }
    if (total > INT64_MAX / (K / 16)) return NVFP4_ERR_SHAPE;
    if (!aligned(module_gs, 4) || !aligned(shared_gs, 4) || (counters && !aligned(counters, 4)))
      return NVFP4_ERR_ALIGN;
    // the shared scale is written while module scales are still being read
    const uintptr_t g0 = (uintptr_t)module_gs, g1 = g0 + 4u * (uintptr_t)n_modules;
    const uintptr_t s0 = (uintptr_t)shared_gs;
    if (s0 + 4 > g0 && s0 < g1) return NVFP4_ERR_ALIAS;
    return hip_status(nvfp4::launch_harmonize(scales, module_gs, module_rows, n_modules, K, shared_gs,
                                              counters, (hipStream_t)stream));
  } catch (...) {
    return NVFP4_ERR_HIP;
  }
}

const char* nvfp4_status_string(int32_t status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "invalid shape";
    case NVFP4_ERR_DTYPE: return "unknown dtype";
    case NVFP4_ERR_MODE: return "unknown scale mode";
    case NVFP4_ERR_ALIGN: return "misaligned pointer or row stride";
    case NVFP4_ERR_WORKSPACE: return "workspace too small";
    case NVFP4_ERR_HIP: return "HIP launch failed";
    case NVFP4_ERR_ALIAS: return "output overlaps an input that is still being read";
    case NVFP4_ERR_TOO_LARGE:
      return "the quantized activations need more than the static scratch of nvfp4_quantize_gemm_no_alloc "
             "(nvfp4_quantize_gemm_no_alloc_max_bytes())";
    default: return "unknown status";
  }
}

int32_t nvfp4_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
