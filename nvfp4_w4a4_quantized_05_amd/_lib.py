"""ctypes binding of ``libnvfp4.so``: argument marshalling only.

Names mirror the C ABI in ``include/nvfp4.h``.  torch supplies device memory
and the current stream; every step of the computation runs in the HIP
library.  There is no fallback: if the library is missing, or a tensor is not
on a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvfp4.so")

NVFP4_OK = 0
IN_F32, IN_BF16 = 0, 1
OUT_F32, OUT_BF16 = 0, 1
SCALE_GIVEN, SCALE_FROM_AMAX = 0, 1
STATUS_NAMES = {0: "NVFP4_OK", 1: "NVFP4_ERR_NULL", 2: "NVFP4_ERR_SHAPE", 3: "NVFP4_ERR_DTYPE",
                4: "NVFP4_ERR_MODE", 5: "NVFP4_ERR_ALIGN", 6: "NVFP4_ERR_WORKSPACE",
                7: "NVFP4_ERR_HIP", 8: "NVFP4_ERR_ALIAS", 9: "NVFP4_ERR_TOO_LARGE"}
EXPORTS = ("nvfp4_quantize", "nvfp4_gemm", "nvfp4_gemm_segmented", "nvfp4_gemm_segmented_gates",
           "nvfp4_quantize_gemm", "nvfp4_gdn_recurrence", "nvfp4_gemm_swiglu_quantize",
           "nvfp4_quantize_gemm_workspace_size", "nvfp4_quantize_gemm_no_alloc",
           "nvfp4_quantize_gemm_no_alloc_max_bytes", "nvfp4_harmonize_fused_scales",
           "nvfp4_gemm_workspace_size", "nvfp4_status_string", "nvfp4_last_hip_error")

_lib = None


class Nvfp4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = load().nvfp4_status_string(status).decode()
        if status == 7:
            msg += f" (hipError {load().nvfp4_last_hip_error()})"
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)}: {msg}")


def load() -> ctypes.CDLL:
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m nvfp4_w4a4_quantized_05_amd.build` (needs hipcc)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.nvfp4_quantize.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, i32, vp]
    lib.nvfp4_quantize.restype = i32
    lib.nvfp4_gemm.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, vp, i32, i64, vp, sz, vp]
    lib.nvfp4_gemm.restype = i32
    lib.nvfp4_gemm_segmented.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.POINTER(i64), i32, i64, i64, vp, i32,
                                         i64, vp, sz, vp]
    lib.nvfp4_gemm_segmented.restype = i32
    lib.nvfp4_gemm_segmented_gates.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.POINTER(i64), i32, i32, vp, vp, i32,
                                               i64, i64, vp, i32, i64, vp, sz, vp]
    lib.nvfp4_gemm_segmented_gates.restype = i32
    lib.nvfp4_gemm_swiglu_quantize.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, vp, vp, vp, vp, i64, vp]
    lib.nvfp4_gemm_swiglu_quantize.restype = i32
    lib.nvfp4_gdn_recurrence.argtypes = [vp, i64, i64, i64, i64, i64, i64, i64, i32, i32, vp, vp, vp, i64, vp, vp,
                                         i32, vp, vp]
    lib.nvfp4_gdn_recurrence.restype = i32
    lib.nvfp4_quantize_gemm.argtypes = [vp, i32, i64, vp, vp, vp, vp, i64, i64, i64, vp, i32, i64, vp, sz, vp]
    lib.nvfp4_quantize_gemm.restype = i32
    lib.nvfp4_quantize_gemm_workspace_size.argtypes = [i64, i64, i64, i32, i32]
    lib.nvfp4_quantize_gemm_workspace_size.restype = sz
    lib.nvfp4_quantize_gemm_no_alloc.argtypes = [vp, i32, i64, vp, vp, vp, vp, i64, i64, i64, vp, i32, i64, vp]
    lib.nvfp4_quantize_gemm_no_alloc.restype = i32
    lib.nvfp4_quantize_gemm_no_alloc_max_bytes.argtypes = []
    lib.nvfp4_quantize_gemm_no_alloc_max_bytes.restype = sz
    lib.nvfp4_harmonize_fused_scales.argtypes = [vp, vp, ctypes.POINTER(i64), i32, i64, vp, vp, vp]
    lib.nvfp4_harmonize_fused_scales.restype = i32
    lib.nvfp4_gemm_workspace_size.argtypes = [i64, i64, i64, i32]
    lib.nvfp4_gemm_workspace_size.restype = sz
    lib.nvfp4_status_string.argtypes = [i32]
    lib.nvfp4_status_string.restype = ctypes.c_char_p
    lib.nvfp4_last_hip_error.argtypes = []
    lib.nvfp4_last_hip_error.restype = i32
    _lib = lib
    return lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, what: str):
    if status != NVFP4_OK:
        raise Nvfp4Error(status, what)


def _need_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("nvfp4 calls take GPU tensors only")


def _u8_matrix(t, shape, what):
    """t must be a contiguous uint8 tensor of exactly `shape`."""
    if t.dtype != torch.uint8 or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous uint8 {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")


def _f32_scalars(t, n, what):
    """t must hold at least n contiguous float32 values (tensor scales)."""
    if t.dtype != torch.float32 or t.numel() < n or not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous float32 with {n} value(s)")


def _out_matrix(out, M, N, out_dtype):
    """out: 2-D, out_dtype, M rows, at least N columns, unit column stride."""
    if out.dtype != out_dtype or out.dim() != 2 or out.stride(1) != 1:
        raise ValueError("out must be 2-D with unit column stride and dtype out_dtype")
    if out.shape[0] != M or out.shape[1] < N:
        raise ValueError(f"out must be [{M}, >= {N}], got {tuple(out.shape)}")


def _operands(a_codes, a_scales, a_gs, w_codes, w_scales, k):
    """Shapes of the two NVFP4 operands; returns (M, N, K)."""
    M = a_codes.shape[0]
    N = w_codes.shape[0]
    K = a_codes.shape[1] * 2 if k is None else k
    if a_codes.dim() != 2 or w_codes.dim() != 2 or K <= 0 or K % 16:
        raise ValueError("codes must be 2-D and K a positive multiple of 16")
    _u8_matrix(a_codes, (M, K // 2), "a_codes")
    _u8_matrix(a_scales, (M, K // 16), "a_scales")
    _u8_matrix(w_codes, (N, K // 2), "w_codes")
    _u8_matrix(w_scales, (N, K // 16), "w_scales")
    _f32_scalars(a_gs, 1, "a_gs")
    return M, N, K


def quantize(x: torch.Tensor, global_scale: torch.Tensor | None = None, *, from_amax: bool | None = None,
             codes: torch.Tensor | None = None, scales: torch.Tensor | None = None, stream=None):
    """NVFP4-encode a 2-D bf16 or fp32 GPU tensor (rows contiguous, any row stride).

    ``global_scale`` is a one-element fp32 GPU tensor: read when it is given
    (calibrated scale), written with RN32(amax/2688) when ``from_amax``
    (default: from_amax = global_scale is None).  Returns (codes, scales, gs).
    """
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    if x.dtype == torch.bfloat16:
        dt = IN_BF16
    elif x.dtype == torch.float32:
        dt = IN_F32
    else:
        raise ValueError(f"unsupported input dtype {x.dtype}")
    rows, cols = x.shape
    if cols % 16:
        raise ValueError("columns must be a multiple of 16")
    if codes is not None:
        _u8_matrix(codes, (rows, cols // 2), "codes")
    if scales is not None:
        _u8_matrix(scales, (rows, cols // 16), "scales")
    if global_scale is not None:
        _f32_scalars(global_scale, 1, "global_scale")
    _need_gpu(x, global_scale, codes, scales)
    if from_amax is None:
        from_amax = global_scale is None
    if global_scale is None:
        global_scale = torch.empty(1, dtype=torch.float32, device=x.device)
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=x.device)
    st = load().nvfp4_quantize(_ptr(x), dt, rows, cols, x.stride(0), _ptr(codes), _ptr(scales),
                               _ptr(global_scale), SCALE_FROM_AMAX if from_amax else SCALE_GIVEN,
                               _stream(stream))
    _check(st, "nvfp4_quantize")
    return codes, scales, global_scale


def gemm(a_codes, a_scales, a_gs, w_codes, w_scales, w_gs, *, out_dtype=torch.float32,
         out: torch.Tensor | None = None, k: int | None = None, stream=None):
    """y[M, N] = RN32(g_a g_w) deq(A) deq(W)^T from NVFP4 A [M, K] and W [N, K]."""
    M, N, K = _operands(a_codes, a_scales, a_gs, w_codes, w_scales, k)
    _f32_scalars(w_gs, 1, "w_gs")
    od = {torch.float32: OUT_F32, torch.bfloat16: OUT_BF16}[out_dtype]
    if out is not None:
        _out_matrix(out, M, N, out_dtype)
    _need_gpu(a_codes, a_scales, a_gs, w_codes, w_scales, w_gs, out)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a_codes.device)
    lib = load()
    ws_bytes = lib.nvfp4_gemm_workspace_size(M, N, K, od)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=a_codes.device) if ws_bytes else None
    st = lib.nvfp4_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(a_gs), _ptr(w_codes), _ptr(w_scales),
                        _ptr(w_gs), M, N, K, _ptr(out), od, out.stride(0), _ptr(ws), ws_bytes,
                        _stream(stream))
    _check(st, "nvfp4_gemm")
    return out


def gemm_segmented(a_codes, a_scales, a_gs, w_codes, w_scales, module_gs, module_rows, *,
                   out_dtype=torch.float32, out: torch.Tensor | None = None, k: int | None = None, stream=None):
    """One GEMM over modules concatenated along N (module_rows rows each): the
    columns of module i are RN32(g_a g_i) deq(A) deq(W_i)^T, g_i = module_gs[i]."""
    rows = [int(r) for r in module_rows]
    M, N, K = _operands(a_codes, a_scales, a_gs, w_codes, w_scales, k)
    if sum(rows) != N or module_gs.numel() != len(rows) or module_gs.dtype != torch.float32:
        raise ValueError("module_rows must sum to the weight rows, one float32 scale per module")
    od = {torch.float32: OUT_F32, torch.bfloat16: OUT_BF16}[out_dtype]
    if out is not None:
        _out_matrix(out, M, N, out_dtype)
    _need_gpu(a_codes, a_scales, a_gs, w_codes, w_scales, module_gs, out)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a_codes.device)
    lib = load()
    ws_bytes = lib.nvfp4_gemm_workspace_size(M, N, K, od)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=a_codes.device) if ws_bytes else None
    host_rows = (ctypes.c_int64 * len(rows))(*rows)
    st = lib.nvfp4_gemm_segmented(_ptr(a_codes), _ptr(a_scales), _ptr(a_gs), _ptr(w_codes), _ptr(w_scales),
                                  _ptr(module_gs.contiguous()), host_rows, len(rows), M, K, _ptr(out), od,
                                  out.stride(0), _ptr(ws), ws_bytes, _stream(stream))
    _check(st, "nvfp4_gemm_segmented")
    return out


def gemm_segmented_gates(a_codes, a_scales, a_gs, w_codes, w_scales, module_gs, module_rows, *,
                         decay_module: int = -1, a_log: torch.Tensor | None = None,
                         dt_bias: torch.Tensor | None = None, write_module: int = -1,
                         out_dtype=torch.float32, out: torch.Tensor | None = None, stream=None):
    """gemm_segmented whose epilogue turns module `decay_module` into the decay
    gate -exp(a_log) softplus(v + dt_bias) and module `write_module` into
    sigmoid(v) (-1: none)."""
    rows = [int(r) for r in module_rows]
    M, N, K = _operands(a_codes, a_scales, a_gs, w_codes, w_scales, None)
    if sum(rows) != N or module_gs.numel() != len(rows) or module_gs.dtype != torch.float32:
        raise ValueError("module_rows must sum to the weight rows, one float32 scale per module")
    if decay_module >= 0:
        for t in (a_log, dt_bias):
            if t is None or t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != rows[decay_module]:
                raise ValueError("a_log and dt_bias: contiguous float32, one per decay-module row")
    od = {torch.float32: OUT_F32, torch.bfloat16: OUT_BF16}[out_dtype]
    if out is not None:
        _out_matrix(out, M, N, out_dtype)
    _need_gpu(a_codes, a_scales, a_gs, w_codes, w_scales, module_gs, a_log, dt_bias, out)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a_codes.device)
    lib = load()
    ws_bytes = lib.nvfp4_gemm_workspace_size(M, N, K, od)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=a_codes.device) if ws_bytes else None
    host_rows = (ctypes.c_int64 * len(rows))(*rows)
    st = lib.nvfp4_gemm_segmented_gates(_ptr(a_codes), _ptr(a_scales), _ptr(a_gs), _ptr(w_codes), _ptr(w_scales),
                                        _ptr(module_gs.contiguous()), host_rows, len(rows), decay_module,
                                        _ptr(a_log), _ptr(dt_bias), write_module, M, K, _ptr(out), od,
                                        out.stride(0), _ptr(ws), ws_bytes, _stream(stream))
    _check(st, "nvfp4_gemm_segmented_gates")
    return out


def gemm_swiglu_quantize(a_codes, a_scales, a_gs, w_codes, w_scales, w_gs, h_gs, *, codes=None, scales=None,
                         h: torch.Tensor | None = None, stream=None):
    """h = silu(gate) * up of the gate/up GEMM (W = [gate; up], 2F rows),
    quantized with tensor scale h_gs in the epilogue.  Returns (codes
    [M, F/2], scales [M, F/16], h_gs); h [M, >= F] fp32 is filled if given."""
    M, N, K = _operands(a_codes, a_scales, a_gs, w_codes, w_scales, None)
    if N % 2:
        raise ValueError("the gate/up weight has 2F rows")
    F = N // 2
    _f32_scalars(w_gs, 1, "w_gs")
    _f32_scalars(h_gs, 1, "h_gs")
    _need_gpu(a_codes, a_scales, a_gs, w_codes, w_scales, w_gs, h_gs, codes, scales, h)
    if codes is None:
        codes = torch.empty((M, F // 2), dtype=torch.uint8, device=a_codes.device)
    if scales is None:
        scales = torch.empty((M, F // 16), dtype=torch.uint8, device=a_codes.device)
    if codes.shape != (M, F // 2) or scales.shape != (M, F // 16) or not codes.is_contiguous() \
            or not scales.is_contiguous():
        raise ValueError("codes [M, F/2] and scales [M, F/16], contiguous")
    if h is not None and (h.dtype != torch.float32 or h.dim() != 2 or h.shape[0] != M or h.stride(1) != 1):
        raise ValueError("h must be float32 [M, >= F] with unit column stride")
    st = load().nvfp4_gemm_swiglu_quantize(_ptr(a_codes), _ptr(a_scales), _ptr(a_gs), _ptr(w_codes),
                                           _ptr(w_scales), _ptr(w_gs), M, F, K, _ptr(h_gs), _ptr(codes),
                                           _ptr(scales), _ptr(h), h.stride(0) if h is not None else 0,
                                           _stream(stream))
    _check(st, "nvfp4_gemm_swiglu_quantize")
    return codes, scales, h_gs


def gdn_recurrence(x: torch.Tensor, *, q_col: int, k_col: int, v_col: int, g_col: int, beta_col: int,
                   n_qk_heads: int, n_v_heads: int, state_in: torch.Tensor | None = None,
                   state_out: torch.Tensor | None = None, o: torch.Tensor | None = None,
                   state_norms: torch.Tensor | None = None, snap_steps: torch.Tensor | None = None,
                   snaps: torch.Tensor | None = None, stream=None):
    """Gated DeltaNet recurrence over the T rows of x (fp32 [T, ldx]: q, k,
    v, g, beta at the given columns; v_col = -1 reads v as zero).  Writes
    whichever of state_out [Hv,128,128], o [T, >= Hv*128], state_norms
    [T, Hv] and snaps [n, Hv, 128, 128] (at int32 snap_steps) are given."""
    _need_gpu(x, state_in, state_out, o, state_norms, snap_steps, snaps)
    if x.dim() != 2 or x.dtype != torch.float32 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D float32 tensor with unit column stride")
    T = x.shape[0]
    st_shape = (n_v_heads, 128, 128)
    for t in (state_in, state_out):
        if t is not None and (t.shape != st_shape or t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("states must be contiguous float32 [n_v_heads, 128, 128]")
    if o is not None and (o.dtype != torch.float32 or o.dim() != 2 or o.shape[0] != T or o.stride(1) != 1):
        raise ValueError("o must be float32 [T, >= n_v_heads*128] with unit column stride")
    if state_norms is not None and (state_norms.shape != (T, n_v_heads) or state_norms.dtype != torch.float32
                                    or not state_norms.is_contiguous()):
        raise ValueError("state_norms must be contiguous float32 [T, n_v_heads]")
    n_snaps = 0
    if snap_steps is not None:
        n_snaps = snap_steps.numel()
        if snap_steps.dtype != torch.int32 or snaps is None or snaps.shape != (n_snaps, *st_shape) \
                or snaps.dtype != torch.float32 or not snaps.is_contiguous():
            raise ValueError("snap_steps int32 [n] with snaps float32 [n, n_v_heads, 128, 128]")
    st = load().nvfp4_gdn_recurrence(_ptr(x), x.stride(0), q_col, k_col, v_col, g_col, beta_col, T, n_qk_heads,
                                     n_v_heads, _ptr(state_in), _ptr(state_out), _ptr(o),
                                     o.stride(0) if o is not None else 0, _ptr(state_norms),
                                     _ptr(snap_steps), n_snaps, _ptr(snaps), _stream(stream))
    _check(st, "nvfp4_gdn_recurrence")
    return state_out


def quantize_gemm(x: torch.Tensor, a_gs: torch.Tensor, w_codes, w_scales, w_gs, *, out_dtype=torch.float32,
                  out: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
    """y = gemm(quantize(x, a_gs), W) in one call (one kernel for decode-sized x)."""
    if x.dim() != 2 or x.stride(1) != 1 or x.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("x must be a 2-D bf16 or fp32 tensor with unit column stride")
    M, K = x.shape
    N = w_codes.shape[0]
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    _u8_matrix(w_codes, (N, K // 2), "w_codes")
    _u8_matrix(w_scales, (N, K // 16), "w_scales")
    _f32_scalars(a_gs, 1, "a_gs")
    _f32_scalars(w_gs, 1, "w_gs")
    dt = IN_BF16 if x.dtype == torch.bfloat16 else IN_F32
    od = {torch.float32: OUT_F32, torch.bfloat16: OUT_BF16}[out_dtype]
    if out is not None:
        _out_matrix(out, M, N, out_dtype)
    if workspace is not None and (workspace.dtype != torch.uint8 or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous uint8 tensor")
    _need_gpu(x, a_gs, w_codes, w_scales, w_gs, out, workspace)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    lib = load()
    ws_bytes = lib.nvfp4_quantize_gemm_workspace_size(M, N, K, dt, od)
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    ws_ptr = _ptr(workspace) if ws_bytes else None
    ws_have = workspace.numel() * workspace.element_size() if (ws_bytes and workspace is not None) else 0
    st = lib.nvfp4_quantize_gemm(_ptr(x), dt, x.stride(0), _ptr(a_gs), _ptr(w_codes), _ptr(w_scales), _ptr(w_gs),
                                 M, N, K, _ptr(out), od, out.stride(0), ws_ptr, ws_have, _stream(stream))
    _check(st, "nvfp4_quantize_gemm")
    return out


def quantize_gemm_no_alloc(x: torch.Tensor, a_gs: torch.Tensor, w_codes, w_scales, w_gs, *,
                           out_dtype=torch.float32, out: torch.Tensor | None = None, stream=None):
    """quantize_gemm without a workspace: the library's static device scratch
    holds the quantized activations (nvfp4_quantize_gemm_no_alloc; calls
    that overlap on one GPU race on it).  Allocates out only if not given."""
    if x.dim() != 2 or x.stride(1) != 1 or x.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("x must be a 2-D bf16 or fp32 tensor with unit column stride")
    M, K = x.shape
    N = w_codes.shape[0]
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    _u8_matrix(w_codes, (N, K // 2), "w_codes")
    _u8_matrix(w_scales, (N, K // 16), "w_scales")
    _f32_scalars(a_gs, 1, "a_gs")
    _f32_scalars(w_gs, 1, "w_gs")
    dt = IN_BF16 if x.dtype == torch.bfloat16 else IN_F32
    od = {torch.float32: OUT_F32, torch.bfloat16: OUT_BF16}[out_dtype]
    if out is not None:
        _out_matrix(out, M, N, out_dtype)
    _need_gpu(x, a_gs, w_codes, w_scales, w_gs, out)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    st = load().nvfp4_quantize_gemm_no_alloc(_ptr(x), dt, x.stride(0), _ptr(a_gs), _ptr(w_codes), _ptr(w_scales),
                                             _ptr(w_gs), M, N, K, _ptr(out), od, out.stride(0), _stream(stream))
    _check(st, "nvfp4_quantize_gemm_no_alloc")
    return out


def harmonize_fused_scales(scales: torch.Tensor, module_gs: torch.Tensor, module_rows, k: int, *,
                           shared_gs: torch.Tensor | None = None, counters: torch.Tensor | None = None,
                           stream=None):
    """Rescale (in place) the block scales of modules concatenated along N to
    the shared tensor scale g* = max(module_gs).  Returns (shared_gs, counters)."""
    _need_gpu(scales, module_gs, shared_gs, counters)
    rows = (ctypes.c_int64 * len(module_rows))(*[int(r) for r in module_rows])
    if shared_gs is None:
        shared_gs = torch.empty(1, dtype=torch.float32, device=scales.device)
    if counters is None:
        counters = torch.zeros(2, dtype=torch.int32, device=scales.device)
    st = load().nvfp4_harmonize_fused_scales(_ptr(scales), _ptr(module_gs), rows, len(module_rows), k,
                                              _ptr(shared_gs), _ptr(counters), _stream(stream))
    _check(st, "nvfp4_harmonize_fused_scales")
    return shared_gs, counters
