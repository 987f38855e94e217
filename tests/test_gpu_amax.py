"""The amax pass of nvfp4_quantize (tensor scale RN32(amax / 2688)): the
tensor maximum placed in the first chunk, the last (partial) window, and
the middle, at sizes below one window, across many windows per workgroup
(the grid is capped, so large tensors take several passes), with a row
stride, where larger values sit in the padding between rows and must not
count, and for bf16 and fp32 input.  The scale is checked bit-exact against
the oracle's, and the codes of a large case against the oracle's quantize
with that scale."""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_05_amd as nv
from oracle import nvfp4_ref as ref
from tests.gpu_util import assert_quantize_matches_oracle_full, host_f32, need_gpu

pytestmark = pytest.mark.gpu

# (rows, cols, padding columns): one 16-value block; less than one window of
# 4 x 256 chunks; a ragged chunk count; one window per workgroup; several
# passes per workgroup (32768 x 5120 bf16 = 20 M chunks, 1024 workgroups)
SHAPES = [(1, 16, 0), (3, 48, 16), (7, 1040, 0), (129, 4112, 32), (1000, 4096, 0), (32768, 5120, 0),
          (4099, 17408, 48)]


def _case(rows, cols, pad, dtype, where, seed, dev):
    gen = torch.Generator().manual_seed(seed)
    base = torch.randn(rows, cols + pad, generator=gen)
    if pad:
        base[:, cols:] = 1e6          # padding: larger than any value of the tensor
    x_full = base.to(dtype).to(dev)
    x = x_full[:, :cols]
    r, c = {"first": (0, 0), "last": (rows - 1, cols - 1), "middle": (rows // 2, cols // 2 + 3)}[where]
    c = min(c, cols - 1)
    x[r, c] = -4096.5 if dtype == torch.float32 else -4096.0   # the tensor maximum, negative
    return x


@pytest.mark.parametrize("rows,cols,pad", SHAPES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_amax_scale_matches_oracle(rows, cols, pad, dtype):
    dev = need_gpu()
    if dtype == torch.float32 and rows * cols > 1 << 26:
        pytest.skip("fp32 copy of the largest shape is covered by bf16")
    for i, where in enumerate(("first", "last", "middle")):
        print(f"[amax] {rows}x{cols}+{pad} {dtype} max at {where}", flush=True)
        x = _case(rows, cols, pad, dtype, where, seed=rows * 7 + i, dev=dev)
        _, _, g = nv.quantize(x)
        torch.cuda.synchronize()
        xh = host_f32(x)
        want = ref.global_scale(xh)
        assert want == np.float32(4096.5 if dtype == torch.float32 else 4096.0) / np.float32(2688.0)
        got = np.float32(g.item())
        assert got.view(np.uint32) == want.view(np.uint32), (where, got, want)


def test_amax_codes_of_a_strided_layer_input():
    # a 32768 x 5120 bf16 view of rows 5152 wide: codes and scales from the
    # amax-derived tensor scale match the oracle's on every block
    dev = need_gpu()
    x = _case(32768, 5120, 32, torch.bfloat16, "last", seed=11, dev=dev)
    codes, scales, g = nv.quantize(x)
    torch.cuda.synchronize()
    want = ref.global_scale(host_f32(x))
    assert np.float32(g.item()).view(np.uint32) == want.view(np.uint32)
    assert_quantize_matches_oracle_full(x, codes, scales, want, "amax-mode quantize, strided")
