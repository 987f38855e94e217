/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 W4A4 linear-layer library.
 *
 * The format, as the pages on arXiv 2609.04098 ("Why Gated DeltaNet Survives
 * 4-Bit Quantization: NVFP4 W4A4 for the Recurrent Half of a Hybrid 27B LLM")
 * define it: picx.dev summary, "Introduction and Theoretical Foundation" >
 * "Background", item 1 -- each value is a 4-bit E2M1 float, each block of 16
 * consecutive values has one E4M3 scale set to the block's absolute maximum
 * divided by 6, and the tensor has one FP32 scale; anthology record LIT-800,
 * "Standing in the anthology" -- 16-element blocks with an E4M3 scale, where
 * MX uses 32 elements and a power-of-two scale.
 *
 * Exact semantics implemented (the pages leave the arithmetic open; this is
 * the plainest reading, applied bit-exactly):
 *   g      = RN32(amax / 2688), or 1.0 if that is 0          (tensor scale)
 *   s_blk  = E4M3 round-to-nearest-even of blockmax / (6 g), exact real
 *            quotient, saturated at 448 (0x7E); subnormals kept; 0 allowed
 *   code   = sign(x) << 3 | E2M1 round-to-nearest-even of |x| / (s_blk g),
 *            exact real quotient, saturated at 6; zero scale -> magnitude 0
 *   deq(x) = E2M1(code) * E4M3(s_blk) * g
 * Codes are packed two per byte (even column in the low nibble) into a
 * row-major [rows x cols/2] array; scales are a row-major [rows x cols/16]
 * array of E4M3 ("fn" variant: bias 7, no infinity, 0x7F = NaN) bytes.
 * Blocks run along the contraction dimension K of both GEMM operands, so
 * weights are stored [N x K] (out x in), K contiguous.
 *
 * Conventions shared by every call:
 *   - Every tensor pointer is a DEVICE pointer (hipMalloc'd or from torch);
 *     host pointers are named as such.  The caller owns every buffer; the
 *     library allocates nothing and keeps no mutable global state.
 *   - Calls enqueue work on `stream` (a hipStream_t, passed as void*; NULL is
 *     the default stream) and return without synchronizing.  Tensor scales
 *     stay on the device: no host<->device copy happens inside a call.
 *   - All argument checks run before any HIP call.  A failed check returns
 *     its status and enqueues nothing.  A failed kernel launch returns
 *     NVFP4_ERR_HIP (see nvfp4_last_hip_error).  Faults inside a kernel
 *     surface asynchronously through HIP, as for any kernel.
 *   - Rows == 0 is a valid no-op.  Exceptions never cross the ABI.  Calls on
 *     different streams are independent; calls that write the same buffers
 *     concurrently race.
 *   - Bit-exactness against the exact-real definition above holds for tensor
 *     scales g in [2^-100, 2^100] (amax in [2^-88, 2^111] for computed
 *     scales) and finite inputs.  Non-finite inputs give unspecified codes.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef NVFP4_API
#define NVFP4_API __attribute__((visibility("default")))
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,      /* a required pointer is NULL                       */
  NVFP4_ERR_SHAPE = 2,     /* bad size: negative, K/cols % 16 != 0, ld < cols */
  NVFP4_ERR_DTYPE = 3,     /* unknown input/output dtype code                  */
  NVFP4_ERR_MODE = 4,      /* unknown scale mode                               */
  NVFP4_ERR_ALIGN = 5,     /* a pointer is not aligned as documented           */
  NVFP4_ERR_WORKSPACE = 6, /* workspace too small                              */
  NVFP4_ERR_HIP = 7,       /* a HIP launch failed; see nvfp4_last_hip_error()  */
  NVFP4_ERR_ALIAS = 8,     /* an output overlaps an input it must not overlap  */
  NVFP4_ERR_TOO_LARGE = 9  /* more than the allocation-free entry point's static
                              scratch (nvfp4_quantize_gemm_no_alloc)         */
} nvfp4_status_t;

typedef enum { NVFP4_IN_F32 = 0, NVFP4_IN_BF16 = 1 } nvfp4_in_t;
typedef enum { NVFP4_OUT_F32 = 0, NVFP4_OUT_BF16 = 1 } nvfp4_out_t;
typedef enum { NVFP4_SCALE_GIVEN = 0, NVFP4_SCALE_FROM_AMAX = 1 } nvfp4_scale_mode_t;

/*
 * nvfp4_quantize -- NVFP4 encode of a row-major [rows x cols] tensor
 * (picx.dev summary, "Background", item 1: E2M1 values, one E4M3 scale of
 * blockmax/6 per 16 values, one FP32 tensor scale).
 *
 *   x            device, [rows x ldx] elements of type `in_dtype`
 *                (NVFP4_IN_F32 or NVFP4_IN_BF16); 16-byte aligned, and
 *                ldx * element size a multiple of 16 bytes
 *   rows, cols   rows >= 0; cols > 0 and cols % 16 == 0
 *   ldx          row stride of x in elements, ldx >= cols
 *   codes        device out, [rows x cols/2] bytes, 8-byte aligned
 *   scales       device out, [rows x cols/16] E4M3 bytes
 *   global_scale device, one float.  NVFP4_SCALE_GIVEN: read (the caller's
 *                positive finite calibrated scale g).  NVFP4_SCALE_FROM_AMAX:
 *                written with g = RN32(amax/2688) (1.0 if that is 0) computed
 *                from x, then used.
 *   mode         nvfp4_scale_mode_t
 *   stream       hipStream_t or NULL
 * FROM_AMAX enqueues four kernels (clear, absolute-max reduction, encode,
 * finalize); GIVEN enqueues one.  Output is deterministic.  rows == 0:
 * nothing is encoded (x, codes and scales may be NULL); FROM_AMAX still
 * writes g = 1.0, the amax of no values being 0, and GIVEN enqueues nothing.
 */
NVFP4_API nvfp4_status_t nvfp4_quantize(const void* x, int32_t in_dtype, int64_t rows, int64_t cols,
                              int64_t ldx, uint8_t* codes, uint8_t* scales,
                              float* global_scale, int32_t mode, void* stream);

/*
 * nvfp4_gemm -- W4A4 linear layer y = (g_a g_w) * deq(A) * deq(W)^T
 * (picx.dev summary, "Background", item 1: both operands NVFP4, multiplied
 * as 4-bit values; the MI355X path dequantizes each E2M1 x E4M3 product
 * exactly to fp16 and accumulates in fp32 on the matrix cores, then applies
 * RN32(g_a g_w) in the epilogue).
 *
 *   a_codes, a_scales  device, A = [M x K] activations in the layout above
 *   a_gs               device, one float: g_a
 *   w_codes, w_scales  device, W = [N x K] weights in the layout above
 *   w_gs               device, one float: g_w
 *   M, N, K            M >= 0, N > 0, K > 0, K % 16 == 0
 *   y                  device out, [M x ldy] of `out_dtype` (NVFP4_OUT_F32 or
 *                      NVFP4_OUT_BF16, round-to-nearest-even); ldy >= N
 *   workspace          device scratch, 16-byte aligned, owned by the caller
 *                      (NULL when nvfp4_gemm_workspace_size() is 0); at least
 *                      nvfp4_gemm_workspace_size(M, N, K, out_dtype) bytes
 *                      are required, else NVFP4_ERR_WORKSPACE.  Its contents
 *                      need no initialisation and are overwritten.  Calls
 *                      that share one workspace must be ordered (one stream).
 * Fast path: K % 128 == 0 and codes/scales base pointers 16-/8-byte aligned;
 * other K % 16 == 0 shapes take a slower generic kernel with the same result.
 * Accuracy: |y - Y| <= 1e-4 * sum_k |a_k w_k| against the exact product for
 * fp32 output (plus half a bf16 ulp of Y for bf16 output).  Deterministic:
 * the same inputs give bit-identical output.
 * Tail split: the fast path gives each workgroup a 256 x 256 output tile, one
 * per CU at a time.  When the tile count leaves the last round of 256 at most
 * a quarter full (4096 x 12384 has 784 tiles: 3 rounds and 16 tiles), each
 * of those last tiles is split over K into 2-8 parts computed side by side;
 * their fp32 partial sums go to the workspace and a second kernel adds them
 * in part order, scales and writes them.  Only these shapes need a workspace.
 */
NVFP4_API nvfp4_status_t nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
                          const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gs,
                          int64_t M, int64_t N, int64_t K, void* y, int32_t out_dtype,
                          int64_t ldy, void* workspace, size_t workspace_bytes, void* stream);

/*
 * nvfp4_gemm_segmented -- one GEMM over modules concatenated along N, each
 * keeping its own tensor scale: output columns of module i are
 * RN32(g_a g_i) * deq(A) * deq(W_i)^T, where deq leaves out the tensor scale.
 * This serves a fused projection (the GDN in-projection: qkv, z and the
 * small a and b gate projections) with exactly the per-module result, with
 * no rescaling of block scales (cctest.ai article "Why Gated DeltaNet Holds
 * Up Under 4-Bit Quantization", "Main findings", last bullet, and LIT-800
 * "Standing in the anthology": a fused kernel that applies one module's
 * tensor scale to all of them mis-scales the others).  The pages repair the
 * mismatch in the checkpoint instead (nvfp4_harmonize_fused_scales); this
 * call is the alternative that moves the per-module scale to the epilogue.
 *
 *   a_codes, a_scales, a_gs   as for nvfp4_gemm
 *   w_codes, w_scales         device, the modules' weights concatenated
 *                             along N, each quantized with its own g_i
 *   module_gs                 device, n_modules floats g_i
 *   module_rows               HOST, n_modules row counts (each >= 0);
 *                             N = their sum, 0 < N <= INT_MAX
 *   n_modules                 1 .. 64
 *   M, K, y, out_dtype, ldy, workspace, workspace_bytes, stream
 *                             as for nvfp4_gemm
 * Same kernels, accuracy and determinism as nvfp4_gemm; nvfp4_gemm is the
 * case n_modules = 1.  NVFP4_ERR_NULL if module_rows is NULL; other errors as
 * for nvfp4_gemm.
 */
NVFP4_API nvfp4_status_t nvfp4_gemm_segmented(const uint8_t* a_codes, const uint8_t* a_scales,
                                              const float* a_gs, const uint8_t* w_codes,
                                              const uint8_t* w_scales, const float* module_gs,
                                              const int64_t* module_rows, int32_t n_modules, int64_t M,
                                              int64_t K, void* y, int32_t out_dtype, int64_t ldy,
                                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * nvfp4_gemm_segmented_gates -- nvfp4_gemm_segmented whose epilogue also
 * evaluates the Gated DeltaNet gates on two of the modules: the log-space
 * decay gate g = -exp(A_log) softplus(a + dt_bias) (picx.dev summary page,
 * "Introduction and Theoretical Foundation" > "Gated DeltaNet Mechanics")
 * and the sigmoid write strength beta = sigmoid(b) (dmarx anthology record
 * LIT-800, "Key takeaways", gates bullet).  With v the module's output
 * RN32(g_a g_i) * deq(A) * deq(W_i)^T (an fp32 value), column j of module
 * `decay_module` becomes -exp(a_log[j]) * softplus(v + dt_bias[j]) and every
 * column of module `write_module` becomes sigmoid(v); other modules are
 * exactly as nvfp4_gemm_segmented writes them.  The gates are evaluated in
 * fp32 with the ROCm device library's expf and log1pf, before the output
 * conversion.
 *
 *   ... as for nvfp4_gemm_segmented, plus
 *   decay_module   index of the decay-gate module (the a projection), or -1
 *   a_log, dt_bias device, module_rows[decay_module] floats each (read);
 *                  may be NULL when decay_module is -1
 *   write_module   index of the write-strength module (the b projection),
 *                  or -1; different from decay_module unless both are -1
 * It splits the same tail tiles as nvfp4_gemm_segmented (the K parts are
 * added first, then the gates applied), so it takes the same workspace.
 * NVFP4_ERR_SHAPE for a module index outside -1 .. n_modules - 1 or equal
 * indices; NVFP4_ERR_NULL / NVFP4_ERR_ALIGN (4 bytes) for the gate
 * parameters; other errors as for nvfp4_gemm_segmented.  Accuracy: the
 * GEMM's bound carried through the gate (|d/dv| <= exp(a_log[j]) for the
 * decay, 1/4 for sigmoid) plus a few fp32 ulp of the gate.
 */
NVFP4_API nvfp4_status_t nvfp4_gemm_segmented_gates(const uint8_t* a_codes, const uint8_t* a_scales,
                                                    const float* a_gs, const uint8_t* w_codes,
                                                    const uint8_t* w_scales, const float* module_gs,
                                                    const int64_t* module_rows, int32_t n_modules,
                                                    int32_t decay_module, const float* a_log,
                                                    const float* dt_bias, int32_t write_module, int64_t M,
                                                    int64_t K, void* y, int32_t out_dtype, int64_t ldy,
                                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * nvfp4_gemm_swiglu_quantize -- the MLP gate/up projection with its output
 * quantized for the down projection in the GEMM's epilogue, so that the
 * gate/up output never goes to memory in bf16.  The pages quantize every
 * linear layer's activations to NVFP4 (picx.dev summary page, "Background",
 * item 1; dmarx anthology record LIT-800, "Key takeaways", recipe bullet);
 * the SwiGLU between the two projections is not on the pages and is this
 * call's assumption: with W = [gate (F rows); up (F rows)] x K,
 *     v = RN32(g_a g_w) deq(A) deq(W)^T          (as nvfp4_gemm, fp32)
 *     h = silu(v_gate) v_up,  silu(x) = x / (1 + exp(-x))
 * in fp32, silu with the hardware exp2 of -x log2(e) and reciprocal
 * and h [M x F] is quantized with the given tensor scale exactly as
 * nvfp4_quantize (GIVEN mode) quantizes fp32 input: the same bytes.
 *
 *   a_codes, a_scales, a_gs   as for nvfp4_gemm (A = [M x K])
 *   w_codes, w_scales, w_gs   the gate and up weights concatenated along N
 *                             ([2F x K], one tensor scale)
 *   M, F, K        M >= 0; F > 0, F % 64 == 0; K > 0, K % 128 == 0;
 *                  M * K / 2 and 2 F * K / 2 below 2^31
 *   h_gs           device, one float: h's tensor scale (read; calibrated)
 *   h_codes, h_scales  device out, [M x F/2] and [M x F/16]
 *   h, ldh         device out [M x ldh] fp32 (ldh >= F, ldh % 4 == 0,
 *                  16-byte aligned), or NULL: h itself
 * Only the streaming kernel has this epilogue; codes and scales of A and W
 * must be 16- and 8-byte aligned (NVFP4_ERR_ALIGN), h_codes 8-byte.
 * Accuracy: v as nvfp4_gemm; h is silu(v_gate) v_up to a few fp32 ulp plus
 * |v_gate| 2^-23 relative (the rounding of v_gate log2(e)); the quantization
 * is exact for that fp32 h.
 */
NVFP4_API nvfp4_status_t nvfp4_gemm_swiglu_quantize(const uint8_t* a_codes, const uint8_t* a_scales,
                                                    const float* a_gs, const uint8_t* w_codes,
                                                    const uint8_t* w_scales, const float* w_gs, int64_t M,
                                                    int64_t F, int64_t K, const float* h_gs, uint8_t* h_codes,
                                                    uint8_t* h_scales, float* h, int64_t ldh, void* stream);

/*
 * nvfp4_gdn_recurrence -- the Gated DeltaNet recurrence of one layer over T
 * tokens, fp32 state (picx.dev summary page, "Introduction and Theoretical
 * Foundation" > "Gated DeltaNet Mechanics", the recurrence as printed there):
 * per value head a state S [128 x 128] (d_k x d_v), and per token t
 *     S_t = alpha_t S_{t-1} + beta_t khat_t (v_t - S_{t-1}^T khat_t)^T,
 *     o_t = S_t^T qhat_t / sqrt(128),
 * with alpha_t = exp(g_t) from the log-space decay gate, beta_t the write
 * strength, and qhat, khat the L2-normalized q, k of the head (divided by
 * max(|.|, 1e-6)).  It consumes the projection rows the fused GDN
 * in-projection writes (nvfp4_gemm_segmented_gates, fp32 output).
 *
 *   x           device, [T x ldx] fp32, one row per token (read);
 *               0 < ldx < 2^23 (NVFP4_ERR_SHAPE otherwise)
 *   q_col, k_col   first column of q / k: n_qk_heads heads of 128 values
 *   v_col       first column of v: n_v_heads heads of 128; -1 reads v as 0
 *               (the recurrence then carries a state perturbation alone)
 *   g_col, beta_col   first column of the n_v_heads decay gates g (log of
 *               alpha) / write strengths beta
 *   T           tokens, 0 .. INT_MAX (0: nothing is enqueued)
 *   n_qk_heads, n_v_heads   value head h reads q/k head
 *               h * n_qk_heads / n_v_heads; n_v_heads % n_qk_heads == 0,
 *               n_v_heads <= 65535
 *   state_in    device [n_v_heads x 128 x 128] fp32 (i = d_k row major), or
 *               NULL for zeros (read)
 *   state_out   device, same layout, or NULL: S_T (written; with T = 0 the
 *               start state, zeros without state_in)
 *   o           device [T x ldo] fp32, head h at columns 128 h, or NULL
 *   state_norms device [T x n_v_heads] fp32 or NULL: |S_t|_F^2 per head
 *   snap_steps, n_snaps, snaps   device: n_snaps strictly increasing token
 *               indices in [0, T) (int32) and [n_snaps x n_v_heads x 128 x
 *               128] fp32 out: S_t after those tokens (a step not above the
 *               previous one, or not below T, is skipped: its slot is not
 *               written)
 * Column ranges must lie within ldx (NVFP4_ERR_SHAPE); pointers 4-byte
 * aligned (NVFP4_ERR_ALIGN).  The columns of each state are independent and
 * are split over workgroups (8 per value head; one per head when
 * state_norms is asked for), each running the tokens in order; the per-token
 * sums are fixed-order, so results are reproducible.  Accuracy: a token
 * adds at most (128 + 16) 2^-24 M_t of rounding error, M_t = max over s <= t
 * of |S_s|_F + beta_s |v_s|, and the update carries the earlier error
 * through alpha I - beta khat khat^T, of spectral norm c_t = max(alpha_t,
 * |alpha_t - beta_t|) <= 1: e_t <= c_t e_{t-1} + (128 + 16) 2^-24 M_t, at most
 * t (128 + 16) 2^-24 M_t.
 */
NVFP4_API nvfp4_status_t nvfp4_gdn_recurrence(const float* x, int64_t ldx, int64_t q_col, int64_t k_col,
                                              int64_t v_col, int64_t g_col, int64_t beta_col, int64_t T,
                                              int32_t n_qk_heads, int32_t n_v_heads, const float* state_in,
                                              float* state_out, float* o, int64_t ldo, float* state_norms,
                                              const int32_t* snap_steps, int32_t n_snaps, float* snaps,
                                              void* stream);

/*
 * nvfp4_quantize_gemm -- quantize the activations with a given (calibrated)
 * tensor scale and multiply: y = nvfp4_gemm(nvfp4_quantize(x, a_gs), W), in
 * one call.  The activation quantization and the linear layer are the ones
 * of nvfp4_quantize (GIVEN mode) and nvfp4_gemm (picx.dev summary,
 * "Background", item 1); the pages' recipe calibrates the activation scales
 * offline (LIT-800, "Key takeaways", recipe bullet), which is what makes the
 * scale a given input here.
 *
 * For decode-sized bf16 inputs (1 <= M <= 2, K % 256 == 0, K <= 8192, and
 * N, K small enough that nvfp4_quantize_gemm_workspace_size() returns 0)
 * one kernel does both: every workgroup quantizes the activations of its K
 * range into LDS while its weight loads are in flight, which saves the
 * quantize launch of a decode step.  Other shapes quantize into the
 * caller's workspace, then run the GEMM.  Either way the output is
 * bit-identical to nvfp4_quantize followed by nvfp4_gemm.
 *
 *   x                 device, M x K activations, bf16 (NVFP4_IN_BF16) or fp32
 *                     (NVFP4_IN_F32), row stride ldx >= K elements; 16-byte
 *                     aligned rows (ldx * element size % 16 == 0)
 *   a_gs              device, one float: the activations' tensor scale (read)
 *   w_codes, w_scales, w_gs, N, K, y, out_dtype, ldy   as for nvfp4_gemm;
 *                     the one-kernel path needs w_codes 16-byte and w_scales
 *                     8-byte aligned (else NVFP4_ERR_ALIGN)
 *   workspace         device scratch of nvfp4_quantize_gemm_workspace_size()
 *                     bytes (16-byte aligned; may be NULL when that is 0)
 * Errors as for nvfp4_quantize and nvfp4_gemm; NVFP4_ERR_WORKSPACE if the
 * workspace is too small.
 */
NVFP4_API nvfp4_status_t nvfp4_quantize_gemm(const void* x, int32_t in_dtype, int64_t ldx, const float* a_gs,
                                             const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gs,
                                             int64_t M, int64_t N, int64_t K, void* y, int32_t out_dtype,
                                             int64_t ldy, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace nvfp4_quantize_gemm needs: 0 when one kernel does both
 * steps, else M*K/2 rounded up to 256 plus M*K/16 (codes, then scales). */
NVFP4_API size_t nvfp4_quantize_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int32_t in_dtype,
                                                    int32_t out_dtype);

/*
 * nvfp4_quantize_gemm_no_alloc -- nvfp4_quantize_gemm for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It takes no workspace: where
 * nvfp4_quantize_gemm would quantize the activations into the caller's
 * workspace, this call uses a static device array of
 * nvfp4_quantize_gemm_no_alloc_max_bytes() bytes (4 MiB) that the library
 * holds on every GPU it runs on until the process ends.  It calls no
 * hipMalloc, hipFree or allocating library routine; on its first call on a
 * device it looks up that device's copy of the array (hipGetSymbolAddress).
 *
 * Arguments, layouts and results are those of nvfp4_quantize_gemm (same
 * kernels, same bytes) without workspace and workspace_bytes.  The caller
 * still owns x, y and the weights.
 *
 * Limit: nvfp4_quantize_gemm_workspace_size(M, N, K, in_dtype, out_dtype)
 * (about M * K * 9/16 bytes) must not exceed the array: 64 rows up to
 * K = 116,496, 910 rows at K = 8192, 1,456 rows at K = 5120.  Larger
 * problems return NVFP4_ERR_TOO_LARGE before anything is enqueued.  The array keeps the last call's contents (nothing in it has to
 * start at zero: every call writes what it reads).  All calls on one GPU
 * share it, so calls that overlap in time on one GPU (several streams or
 * host threads without ordering between them) race on it and may give wrong
 * results; calls ordered on one stream are safe.
 */
NVFP4_API nvfp4_status_t nvfp4_quantize_gemm_no_alloc(const void* x, int32_t in_dtype, int64_t ldx,
                                                      const float* a_gs, const uint8_t* w_codes,
                                                      const uint8_t* w_scales, const float* w_gs, int64_t M,
                                                      int64_t N, int64_t K, void* y, int32_t out_dtype,
                                                      int64_t ldy, void* stream);

/* Bytes of the static scratch of nvfp4_quantize_gemm_no_alloc, per GPU. */
NVFP4_API size_t nvfp4_quantize_gemm_no_alloc_max_bytes(void);

/*
 * nvfp4_harmonize_fused_scales -- re-express the block scales of modules
 * that are concatenated along N into one fused weight, each quantized with
 * its own tensor scale g_i, under one shared tensor scale g* = max_i g_i
 * (cctest.ai article "Why Gated DeltaNet Holds Up Under 4-Bit
 * Quantization", "Main findings", last bullet: fusing independently
 * calibrated GDN projections into one GEMM creates a global-scale mismatch,
 * and the released checkpoint is pre-harmonized; LIT-800 "Standing in the
 * anthology": the fused kernels computed the decay and write gates with
 * mis-scaled weights).  The procedure itself is not on the pages; this call
 * implements: every block scale s of module i becomes
 * E4M3_RNE(E4M3(s) * g_i / g*) (exact real quotient, saturated); codes are
 * left unchanged.  Afterwards a single nvfp4_gemm with w_gs = shared_gs
 * serves the fused weight.
 *
 *   scales       device, in/out, [sum(module_rows) x K/16] E4M3 bytes,
 *                modules concatenated along N in order
 *   module_gs    device, n_modules floats g_i (positive, finite)
 *   module_rows  HOST, n_modules row counts (each >= 0)
 *   n_modules    1 .. 64
 *   K            K > 0, K % 16 == 0
 *   shared_gs    device out, one float: g*; must not overlap module_gs
 *                (NVFP4_ERR_ALIAS)
 *   counters     device out or NULL, two uint32: [0] blocks whose rescale is
 *                inexact (E4M3(s') g* != E4M3(s) g_i), [1] nonzero input
 *                scales whose result has a zero exponent field (subnormal
 *                or zero)
 * Enqueues two kernels (clear counters + rescale).
 */
NVFP4_API nvfp4_status_t nvfp4_harmonize_fused_scales(uint8_t* scales, const float* module_gs,
                                            const int64_t* module_rows, int32_t n_modules,
                                            int64_t K, float* shared_gs, uint32_t* counters,
                                            void* stream);

/* Bytes of workspace nvfp4_gemm, nvfp4_gemm_segmented and
 * nvfp4_gemm_segmented_gates need for this
 * shape: the partial sums of the split tail tiles (256 KiB per tile and
 * part), 0 for every shape without a tail split (out_dtype does not change
 * it).  4096 x 12384 x 5120 needs 32 MiB; the 32K-token projections, the
 * decode shapes and the small shapes need none. */
NVFP4_API size_t nvfp4_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int32_t out_dtype);

/* Static description of a status code; never NULL. */
NVFP4_API const char* nvfp4_status_string(int32_t status);

/* hipError_t of the most recent failed launch on the calling thread (0 if none). */
NVFP4_API int32_t nvfp4_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
