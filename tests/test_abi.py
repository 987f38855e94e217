"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching HIP."""
import ctypes
import os
import re

import pytest

from nvfp4_w4a4_quantized_05_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")

OK, NULL, SHAPE, DTYPE, MODE, ALIGN, WORKSPACE, HIP, ALIAS, TOO_LARGE = range(10)

# Fake, never-dereferenced device addresses: every call below must fail
# validation before it would launch anything.
P16 = ctypes.c_void_p(0x10000)
P_ODD = ctypes.c_void_p(0x10001)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"NVFP4_API\s+[\w\s\*]+?\b(nvfp4_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert names == sorted(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_header_status_codes_match_binding():
    text = open(HEADER).read()
    codes = dict((k, int(v)) for k, v in re.findall(r"(NVFP4_ERR_\w+|NVFP4_OK)\s*=\s*(\d+)", text))
    for num, name in _lib.STATUS_NAMES.items():
        assert codes[name] == num


def test_status_strings(lib):
    for s in range(10):
        assert lib.nvfp4_status_string(s) != b"unknown status"
    assert lib.nvfp4_status_string(99) == b"unknown status"
    assert lib.nvfp4_last_hip_error() == 0


def q(lib, x=P16, dt=1, rows=4, cols=32, ldx=32, codes=P16, scales=P16, gs=P16, mode=0):
    return lib.nvfp4_quantize(x, dt, rows, cols, ldx, codes, scales, gs, mode, None)


def test_quantize_rejects_bad_arguments(lib):
    assert q(lib, dt=2) == DTYPE
    assert q(lib, mode=7) == MODE
    assert q(lib, cols=24, ldx=24) == SHAPE
    assert q(lib, cols=0, ldx=0) == SHAPE
    assert q(lib, rows=-1) == SHAPE
    assert q(lib, ldx=16) == SHAPE
    assert q(lib, x=None) == NULL
    assert q(lib, codes=None) == NULL
    assert q(lib, scales=None) == NULL
    assert q(lib, gs=None) == NULL
    assert q(lib, x=P_ODD) == ALIGN
    assert q(lib, ldx=36) == ALIGN            # bf16 row stride of 72 bytes
    assert q(lib, codes=ctypes.c_void_p(0x10004)) == ALIGN
    assert q(lib, rows=0, x=None, codes=None, scales=None, gs=None) == OK   # empty: no-op
    # empty with the scale from amax: g = 1.0 is still written, so it must be valid
    assert q(lib, rows=0, x=None, codes=None, scales=None, gs=None, mode=1) == NULL
    assert q(lib, rows=0, x=None, codes=None, scales=None, gs=P_ODD, mode=1) == ALIGN
    assert lib.nvfp4_last_hip_error() == 0


def g(lib, M=4, N=8, K=32, y=P16, od=0, ldy=8, ptrs=None, ws_bytes=0):
    p = ptrs or [P16] * 6
    return lib.nvfp4_gemm(*p, M, N, K, y, od, ldy, None, ws_bytes, None)


def test_gemm_rejects_bad_arguments(lib):
    assert g(lib, od=3) == DTYPE
    assert g(lib, K=40) == SHAPE
    assert g(lib, K=0) == SHAPE
    assert g(lib, N=0, ldy=0) == SHAPE
    assert g(lib, M=-2) == SHAPE
    assert g(lib, ldy=4) == SHAPE
    assert g(lib, M=1 << 40) == SHAPE
    for i in range(6):
        p = [P16] * 6
        p[i] = None
        assert g(lib, ptrs=p) == NULL
    assert g(lib, y=None) == NULL
    assert g(lib, y=ctypes.c_void_p(0x10002), od=0) == ALIGN
    assert g(lib, M=0, y=None, ptrs=[None] * 6) == OK
    assert lib.nvfp4_gemm_workspace_size(64, 12288, 5120, 0) == 0


TILE_PART = 256 * 256 * 4  # fp32 partial sums of one 256 x 256 tile and K part


@pytest.mark.parametrize("shape,want", [
    # 784 tiles of 256 x 256: 3 rounds of 256 and 16 tiles, split into 8 parts
    ((4096, 12384, 5120, 0), 16 * 8 * TILE_PART),
    ((4096, 12384, 5120, 1), 16 * 8 * TILE_PART),          # output type does not matter
    ((4059, 12334, 2944, 1), 16 * 5 * TILE_PART),          # 23 K steps: 5 parts of >= 4 steps
    ((4096, 12384, 1024, 0), 16 * 2 * TILE_PART),          # 8 K steps: 2 parts
    ((4096, 12384, 768, 0), 0),                            # 6 K steps: too short to split
    ((4096, 12384, 5120 + 16, 0), 0),                      # K not in whole 128-value steps
    ((4352, 4096, 5120, 0), 16 * 8 * TILE_PART),           # 272 tiles: 16 over one round
    ((2048, 8448 + 256 * 8, 5120, 0), 0),                  # 8 x 41 = 328 tiles: last round 72 > 64
    ((4096, 4096, 5120, 0), 0),                            # exactly one round
    ((4096, 4096 - 256, 5120, 0), 0),                      # fewer tiles than one round
    ((32768, 12384, 5120, 1), 0),                          # the 32K in-projection: 128-tile last round
    ((32768, 34816, 5120, 1), 0), ((32768, 5120, 17408, 1), 0), ((32768, 5120, 4096, 1), 0),
])
def test_gemm_workspace_size_is_the_tail_split(lib, shape, want):
    """nvfp4_gemm_workspace_size: the fp32 partial sums of the split tail
    tiles (tail tiles x parts x 256 KiB), 0 for shapes without a split."""
    assert lib.nvfp4_gemm_workspace_size(*shape) == want


def test_gemm_tail_split_needs_its_workspace(lib):
    """A shape with a tail split: too little workspace, a NULL or misaligned
    workspace are refused before any HIP call, by the plain, segmented and
    gated calls alike."""
    M, N, K = 4096, 12384, 5120
    need = lib.nvfp4_gemm_workspace_size(M, N, K, 0)
    assert need > 0
    p = [P16] * 6
    assert lib.nvfp4_gemm(*p, M, N, K, P16, 0, N, None, need - 1, None) == WORKSPACE
    assert lib.nvfp4_gemm(*p, M, N, K, P16, 0, N, None, 0, None) == WORKSPACE
    assert lib.nvfp4_gemm(*p, M, N, K, P16, 0, N, None, need, None) == NULL
    assert lib.nvfp4_gemm(*p, M, N, K, P16, 0, N, ctypes.c_void_p(0x10008), need, None) == ALIGN
    rows = (ctypes.c_int64 * 1)(N)
    assert lib.nvfp4_gemm_segmented(*[P16] * 5, P16, rows, 1, M, K, P16, 0, N, None, 0, None) == WORKSPACE
    rows3 = (ctypes.c_int64 * 3)(12288, 48, 48)
    assert lib.nvfp4_gemm_segmented_gates(*[P16] * 5, P16, rows3, 3, 1, P16, P16, 2, M, K, P16, 0, N,
                                          None, 0, None) == WORKSPACE
    assert lib.nvfp4_gemm_segmented_gates(*[P16] * 5, P16, rows3, 3, 1, P16, P16, 2, M, K, P16, 0, N,
                                          None, need, None) == NULL
    assert lib.nvfp4_last_hip_error() == 0


def gs_(lib, rows=(8, 0, 4), M=4, K=32, y=P16, od=0, ldy=12, ptrs=None, mgs=P16, n=None, host_rows=True):
    p = ptrs or [P16] * 5
    arr = (ctypes.c_int64 * max(len(rows), 1))(*rows) if host_rows else None
    return lib.nvfp4_gemm_segmented(*p, mgs, arr, len(rows) if n is None else n, M, K, y, od, ldy,
                                    None, 0, None)


def test_gemm_segmented_rejects_bad_arguments(lib):
    assert gs_(lib, host_rows=False) == NULL
    assert gs_(lib, n=0) == SHAPE
    assert gs_(lib, rows=tuple([1] * 65), ldy=65) == SHAPE
    assert gs_(lib, rows=(8, -1, 4)) == SHAPE
    assert gs_(lib, rows=(0, 0), ldy=1) == SHAPE            # N = 0
    assert gs_(lib, rows=(1 << 30, 1 << 30), ldy=1 << 31) == SHAPE   # N > INT_MAX
    assert gs_(lib, ldy=11) == SHAPE                        # ldy < N = 12
    assert gs_(lib, od=2) == DTYPE
    assert gs_(lib, K=24) == SHAPE
    assert gs_(lib, mgs=None) == NULL
    for i in range(5):
        p = [P16] * 5
        p[i] = None
        assert gs_(lib, ptrs=p) == NULL
    assert gs_(lib, mgs=ctypes.c_void_p(0x10002)) == ALIGN
    assert gs_(lib, M=0, y=None, ptrs=[None] * 5, mgs=None) == OK
    assert lib.nvfp4_last_hip_error() == 0


def gg(lib, rows=(8, 4, 2, 2), decay=2, a_log=P16, dt_bias=P16, write=3, M=4, K=32, ldy=16, mgs=P16,
       host_rows=True):
    arr = (ctypes.c_int64 * len(rows))(*rows) if host_rows else None
    return lib.nvfp4_gemm_segmented_gates(P16, P16, P16, P16, P16, mgs, arr, len(rows), decay, a_log, dt_bias,
                                          write, M, K, P16, 0, ldy, None, 0, None)


def test_gemm_segmented_gates_rejects_bad_arguments(lib):
    assert gg(lib, decay=4) == SHAPE                       # module index out of range
    assert gg(lib, write=-2) == SHAPE
    assert gg(lib, decay=3, write=3) == SHAPE              # one module cannot be both gates
    assert gg(lib, a_log=None) == NULL
    assert gg(lib, dt_bias=None) == NULL
    assert gg(lib, a_log=ctypes.c_void_p(0x10002)) == ALIGN
    assert gg(lib, host_rows=False) == NULL
    assert gg(lib, ldy=15) == SHAPE                        # ldy < N = 16
    assert gg(lib, mgs=None) == NULL
    # no decay gate: its parameters may be NULL; M = 0 enqueues nothing
    assert gg(lib, decay=-1, a_log=None, dt_bias=None, M=0) == OK
    assert gg(lib, decay=-1, write=-1, a_log=None, dt_bias=None, M=0) == OK
    assert lib.nvfp4_last_hip_error() == 0


def qg(lib, x=P16, dt=1, ldx=256, a_gs=P16, ptrs=None, M=2, N=64, K=256, y=P16, od=1, ldy=64,
       ws=None, ws_bytes=0):
    p = ptrs or [P16] * 3
    return lib.nvfp4_quantize_gemm(x, dt, ldx, a_gs, *p, M, N, K, y, od, ldy, ws, ws_bytes, None)


def test_quantize_gemm_rejects_bad_arguments_and_sizes_its_workspace(lib):
    assert qg(lib, dt=3) == DTYPE
    assert qg(lib, od=4) == DTYPE
    assert qg(lib, K=40, ldx=40) == SHAPE
    assert qg(lib, ldx=128) == SHAPE
    assert qg(lib, ldy=32) == SHAPE
    assert qg(lib, M=-1) == SHAPE
    assert qg(lib, x=None) == NULL
    assert qg(lib, a_gs=None) == NULL
    for i in range(3):
        p = [P16] * 3
        p[i] = None
        assert qg(lib, ptrs=p) == NULL
    assert qg(lib, y=None) == NULL
    assert qg(lib, x=P_ODD) == ALIGN
    assert qg(lib, ldx=260) == ALIGN                          # bf16 row stride of 520 bytes
    assert qg(lib, M=0, x=None, a_gs=None, ptrs=[None] * 3, y=None) == OK
    # decode-sized: one kernel, no workspace; larger M or K: codes + scales
    assert lib.nvfp4_quantize_gemm_workspace_size(1, 12288, 5120, 1, 1) == 0
    assert lib.nvfp4_quantize_gemm_workspace_size(2, 12384, 4096, 1, 0) == 0
    assert lib.nvfp4_quantize_gemm_workspace_size(3, 12384, 4096, 1, 0) == 3 * 2048 + 3 * 256  # M > 2
    assert lib.nvfp4_quantize_gemm_workspace_size(5, 12384, 4096, 1, 0) == 5 * 2048 + 5 * 256
    assert lib.nvfp4_quantize_gemm_workspace_size(1, 12288, 5120, 0, 1) == 2560 + 320     # fp32 activations
    assert lib.nvfp4_quantize_gemm_workspace_size(40, 12288, 5120, 1, 1) == 40 * 2560 + 40 * 320
    assert lib.nvfp4_quantize_gemm_workspace_size(3, 100, 1040, 0, 1) == 1792 + 3 * 65   # K % 256 != 0
    assert lib.nvfp4_quantize_gemm_workspace_size(2, 12288, 17408, 1, 1) == 17408 + 2 * 1088  # K > 8192
    assert qg(lib, M=40, N=64, K=256, ws_bytes=40 * 128 + 40 * 16 - 1, ws=P16) == WORKSPACE
    assert qg(lib, M=40, N=64, K=256, ws_bytes=1 << 20, ws=None) == NULL
    assert lib.nvfp4_last_hip_error() == 0


def h(lib, scales=P16, mgs=P16, rows=(8, 4), K=32, sgs=ctypes.c_void_p(0x20000), counters=None):
    arr = (ctypes.c_int64 * len(rows))(*rows)
    return lib.nvfp4_harmonize_fused_scales(scales, mgs, arr, len(rows), K, sgs, counters, None)


def test_harmonize_rejects_bad_arguments(lib):
    assert h(lib, scales=None) == NULL
    assert h(lib, mgs=None) == NULL
    assert h(lib, sgs=None) == NULL
    assert h(lib, K=24) == SHAPE
    assert h(lib, rows=()) == SHAPE
    assert h(lib, rows=(1,) * 65) == SHAPE
    assert h(lib, rows=(4, -1)) == SHAPE
    assert h(lib, sgs=ctypes.c_void_p(0x10004)) == ALIAS     # second module scale
    assert h(lib, sgs=ctypes.c_void_p(0x20002)) == ALIGN
    assert h(lib, counters=ctypes.c_void_p(0x30001)) == ALIGN


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        _lib.quantize(x)


def gd(lib, x=P16, ldx=1040, cols=(0, 256, 512, 1024, 1028), T=8, nqk=2, nv_=4, o=None, ldo=0, n_snaps=0,
       steps=None, snaps=None, s_in=None, s_out=None):
    return lib.nvfp4_gdn_recurrence(x, ldx, *cols, T, nqk, nv_, s_in, s_out, o, ldo, None, steps, n_snaps, snaps,
                                    None)


def test_gdn_recurrence_rejects_bad_arguments(lib):
    assert gd(lib, T=-1) == SHAPE
    assert gd(lib, nqk=3) == SHAPE                          # 4 value heads not a multiple of 3
    assert gd(lib, nv_=0) == SHAPE
    assert gd(lib, cols=(0, 256, 512, 1024, 1037)) == SHAPE  # beta columns past ldx
    assert gd(lib, cols=(0, 900, 512, 1024, 1028)) == SHAPE  # k columns past ldx
    assert gd(lib, cols=(0, 256, -2, 1024, 1028)) == SHAPE
    assert gd(lib, o=P16, ldo=511) == SHAPE                  # ldo < 4 * 128
    assert gd(lib, n_snaps=-1) == SHAPE
    assert gd(lib, ldx=1 << 23) == SHAPE                     # rows of 2^23 values or more
    assert gd(lib, x=None) == NULL
    assert gd(lib, n_snaps=2, steps=None, snaps=P16) == NULL
    assert gd(lib, x=ctypes.c_void_p(0x10002)) == ALIGN
    assert gd(lib, s_in=ctypes.c_void_p(0x10002)) == ALIGN
    assert gd(lib, T=0, x=None) == OK                        # nothing to do
    assert gd(lib, T=0, x=None, s_out=P_ODD) == ALIGN        # S_0 would be written there
    assert gd(lib, T=0, cols=(0, 256, -1, 1024, 1028)) == OK  # v = 0 is allowed
    assert lib.nvfp4_last_hip_error() == 0


def sq(lib, ptrs=None, M=4, F=64, K=128, hgs=P16, hc=P16, hs=P16, h=None, ldh=0):
    p = ptrs or [P16] * 6
    return lib.nvfp4_gemm_swiglu_quantize(*p, M, F, K, hgs, hc, hs, h, ldh, None)


def test_gemm_swiglu_quantize_rejects_bad_arguments(lib):
    assert sq(lib, F=96) == SHAPE            # F % 64
    assert sq(lib, K=64) == SHAPE            # K % 128
    assert sq(lib, M=-1) == SHAPE
    assert sq(lib, h=P16, ldh=63) == SHAPE   # ldh < F
    assert sq(lib, M=1 << 20, K=1 << 13) == SHAPE   # M K / 2 >= 2^31
    assert sq(lib, hgs=None) == NULL
    assert sq(lib, hc=None) == NULL
    for i in range(6):
        p = [P16] * 6
        p[i] = None
        assert sq(lib, ptrs=p) == NULL
    assert sq(lib, hc=ctypes.c_void_p(0x10004)) == ALIGN
    assert sq(lib, h=ctypes.c_void_p(0x10008), ldh=64) == ALIGN
    assert sq(lib, h=P16, ldh=66) == ALIGN   # ldh % 4
    assert sq(lib, M=0, ptrs=[None] * 6, hgs=None, hc=None, hs=None) == OK
    assert lib.nvfp4_last_hip_error() == 0


def test_binding_checks_caller_buffers_before_any_call():
    """Buffers the caller passes in (codes, scales, tensor scales, out) are
    checked for dtype, shape and layout before anything reaches the library:
    a smaller out or codes buffer would otherwise be written past its end."""
    import torch
    u8 = lambda *s: torch.zeros(s, dtype=torch.uint8)  # noqa: E731
    f32 = lambda *s: torch.zeros(s, dtype=torch.float32)  # noqa: E731
    x = torch.zeros(4, 32, dtype=torch.bfloat16)
    for kw, msg in ((dict(codes=u8(4, 8)), "codes"), (dict(codes=u8(3, 16)), "codes"),
                    (dict(scales=u8(4, 1)), "scales"), (dict(codes=f32(4, 16)), "codes"),
                    (dict(codes=u8(4, 32)[:, ::2]), "codes"), (dict(global_scale=f32(0)), "global_scale"),
                    (dict(global_scale=torch.zeros(1, dtype=torch.float64)), "global_scale")):
        with pytest.raises(ValueError, match=msg):
            _lib.quantize(x, **kw)
    with pytest.raises(ValueError, match="multiple of 16"):
        _lib.quantize(torch.zeros(4, 24, dtype=torch.bfloat16))
    M, N, K = 8, 48, 64
    a = (u8(M, K // 2), u8(M, K // 16), f32(1))
    w = (u8(N, K // 2), u8(N, K // 16), f32(1))
    for out, msg in ((f32(M - 1, N), "out must be"), (f32(M, N - 1), "out must be"),
                     (torch.zeros(M, N, dtype=torch.bfloat16), "dtype"), (f32(N, M).t(), "stride")):
        with pytest.raises(ValueError, match=msg):
            _lib.gemm(*a, *w, out=out)
        with pytest.raises(ValueError, match=msg):
            _lib.gemm_segmented(*a, *w[:2], f32(2), [16, 32], out=out)
        with pytest.raises(ValueError, match=msg):
            _lib.gemm_segmented_gates(*a, *w[:2], f32(2), [16, 32], out=out)
    with pytest.raises(ValueError, match="a_codes"):
        _lib.gemm(*a, *w, k=2 * K)                       # k disagrees with the codes' width
    with pytest.raises(ValueError, match="w_scales"):
        _lib.gemm(*a, w[0], u8(N, 3), w[2])
    with pytest.raises(ValueError, match="a_gs"):
        _lib.gemm(a[0], a[1], f32(0), *w)
    with pytest.raises(ValueError, match="w_gs"):
        _lib.gemm(*a, w[0], w[1], torch.zeros(1, dtype=torch.float16))
    with pytest.raises(ValueError, match="out must be"):
        _lib.quantize_gemm(torch.zeros(M, K, dtype=torch.bfloat16), f32(1), *w, out=f32(M + 1, N))
    with pytest.raises(ValueError, match="workspace"):
        _lib.quantize_gemm(torch.zeros(M, K, dtype=torch.bfloat16), f32(1), *w, workspace=f32(16))
    with pytest.raises(ValueError, match="h_gs"):
        _lib.gemm_swiglu_quantize(*a, *w, f32(0))
    # well-formed CPU tensors reach the device check, which refuses them
    with pytest.raises(ValueError, match="GPU tensors only"):
        _lib.gemm(*a, *w, out=f32(M, N))


def qgn(lib, x=P16, dt=1, ldx=256, a_gs=P16, M=2, N=64, K=256, y=P16, od=1, ldy=64):
    return lib.nvfp4_quantize_gemm_no_alloc(x, dt, ldx, a_gs, P16, P16, P16, M, N, K, y, od, ldy, None)


def test_quantize_gemm_no_alloc_checks_arguments_and_its_scratch_limit(lib):
    """Same argument checks as nvfp4_quantize_gemm; a problem whose quantized
    activations exceed the static scratch is refused before any HIP call."""
    limit = lib.nvfp4_quantize_gemm_no_alloc_max_bytes()
    assert limit == 4 << 20
    assert qgn(lib, M=0) == OK
    assert qgn(lib, dt=5) == DTYPE and qgn(lib, od=7) == DTYPE
    assert qgn(lib, K=250, ldx=250) == SHAPE and qgn(lib, ldy=10) == SHAPE and qgn(lib, ldx=100) == SHAPE
    assert qgn(lib, x=None) == NULL and qgn(lib, y=None) == NULL and qgn(lib, a_gs=None) == NULL
    assert qgn(lib, x=P_ODD) == ALIGN
    # need = M*K/2 (rounded up to 256) + M*K/16 against the 4 MiB array
    assert lib.nvfp4_quantize_gemm_workspace_size(910, 64, 8192, 1, 1) <= limit
    assert lib.nvfp4_quantize_gemm_workspace_size(911, 64, 8192, 1, 1) > limit
    assert qgn(lib, M=911, K=8192, ldx=8192) == TOO_LARGE
    assert qgn(lib, M=64, K=116512, ldx=116512) == TOO_LARGE
    assert qgn(lib, M=4096, N=4096, K=4096, ldx=4096, ldy=4096) == TOO_LARGE
    assert b"static scratch" in lib.nvfp4_status_string(TOO_LARGE)
