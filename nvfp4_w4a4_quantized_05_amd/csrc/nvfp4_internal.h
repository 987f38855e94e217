// Host-side launchers behind the C ABI.  Arguments are already validated by
// nvfp4_api.cpp; each launcher only enqueues kernels and returns the launch
// status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

hipError_t launch_quantize(const void* x, bool in_bf16, int64_t rows, int64_t cols, int64_t ldx,
                           uint8_t* codes, uint8_t* scales, float* global_scale, bool from_amax,
                           hipStream_t stream);

constexpr int kMaxModules = 64;

// Tensor scales of the weight's output columns.  Column range s (s = 0 ..
// n - 1) is [end[s - 1], end[s]) with end[-1] = 0 and end[n - 1] = N; its
// tensor scale is gs[s] (device).  A plain GEMM is the case n = 1.  Passed
// to the kernels by value (kernel arguments).
struct ColScales {
  const float* gs;
  int n;
  int end[kMaxModules];
  // Gated DeltaNet gate columns (both ranges empty in a plain GEMM).  With
  // v = acc * RN32(g_a g_w): columns [decay_lo, decay_hi) become the decay
  // gate -exp(a_log[j]) softplus(v + dt_bias[j]), j = col - decay_lo, and
  // columns [write_lo, write_hi) the write strength sigmoid(v).
  int decay_lo, decay_hi, write_lo, write_hi;
  const float* a_log;
  const float* dt_bias;
};

// Output of the SwiGLU + quantize epilogue: h = silu(gate) * up of a GEMM
// whose weight rows are [gate (F rows); up (F rows)], quantized with the
// given tensor scale into codes [M x F/2] and scales [M x F/16], and
// optionally written in fp32 to h [M x ldh].
struct SwigluOut {
  const float* gs;
  uint8_t* codes;
  uint8_t* scales;
  float* h;
  int64_t ldh;
  int F;
};

hipError_t launch_gemm_swiglu_quantize(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
                                       const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gs,
                                       int64_t M, int64_t F, int64_t K, const SwigluOut& out, hipStream_t stream);

// Tail split of the large-tile GEMM.  Its workgroups take 256 x 256 output
// tiles, one per CU at a time, so a tile count just above a multiple of 256
// leaves the last round almost empty (4096 x 12384 has 784 tiles: 3 full
// rounds and 16 tiles).  Tiles 0 .. full - 1 are done whole; each of the
// `tail` remaining tiles is split over K into `splits` parts whose fp32
// partial sums go to the workspace, and a second kernel adds the parts in
// part order and writes the output.  splits == 0: no split.
struct SplitTail {
  int full;
  int tail;
  int splits;
  float* part;  // [tail x splits x 64 x 256 x 4] fp32 partial sums (workspace)
};

// The split for a shape on the large-tile kernel (splits == 0 when the last
// round is more than a quarter full, or K is too short to split), and the
// workspace bytes it needs (0 without a split).
SplitTail gemm_split_plan(int64_t M, int64_t N, int64_t K);
size_t gemm_split_workspace_bytes(int64_t M, int64_t N, int64_t K);

// The GEMM; `workspace` (16-byte aligned, workspace_bytes) lets it split the
// last round's tiles when gemm_split_workspace_bytes() > 0 and the
// large-tile kernel runs; NULL / 0 runs without.
hipError_t launch_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
                       const uint8_t* w_codes, const uint8_t* w_scales, const ColScales& cs,
                       int64_t M, int64_t N, int64_t K, void* y, bool out_bf16, int64_t ldy,
                       hipStream_t stream, void* workspace = nullptr, size_t workspace_bytes = 0);

// Decode GEMM with the activation quantization done inside the kernel (bf16
// X, given tensor scale).  Only for shapes where quantize_gemm_fused_fits();
// W pointers 16 / 8 byte aligned, X rows 16 byte aligned.
bool quantize_gemm_fused_fits(int64_t M, int64_t N, int64_t K, bool in_bf16);
hipError_t launch_quantize_gemm_fused(const void* x, bool in_bf16, int64_t ldx, const float* a_gs,
                                      const uint8_t* w_codes, const uint8_t* w_scales, const ColScales& cs,
                                      int64_t M, int64_t N, int64_t K, void* y, bool out_bf16, int64_t ldy,
                                      hipStream_t stream);

// The allocation-free quantize + GEMM keeps the quantized activations in a
// static device array of this many bytes per GPU (nvfp4_noalloc.hip).
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;

// Device address of that array on the current device, looked up with
// hipGetSymbolAddress on the first call per device and kept.
hipError_t no_alloc_scratch(void** ptr);

hipError_t launch_harmonize(uint8_t* scales, const float* module_gs, const int64_t* module_rows,
                            int32_t n_modules, int64_t K, float* shared_gs, uint32_t* counters,
                            hipStream_t stream);

// Gated DeltaNet recurrence over T >= 1 tokens, the columns of each value
// head's state (head dimension 128) split over workgroups; arguments as
// nvfp4_gdn_recurrence, already checked.
hipError_t launch_gdn_recurrence(const float* x, int64_t ldx, int64_t q_col, int64_t k_col, int64_t v_col,
                                 int64_t g_col, int64_t b_col, int64_t T, int n_qk, int n_v, const float* s_in,
                                 float* s_out, float* o, int64_t ldo, float* norms, const int* snap_steps,
                                 int n_snaps, float* snaps, hipStream_t stream);

// S_0 of a recurrence over no tokens: s_out = s_in, or zeros when s_in is
// NULL ([n_v x 128 x 128] fp32; s_in may equal s_out).
hipError_t launch_gdn_start_state(const float* s_in, float* s_out, int n_v, hipStream_t stream);

}  // namespace nvfp4
