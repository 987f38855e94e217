"""The kernels under HIP graph capture: a decode step (quantize with a given
scale, decode GEMM), a prefill step (quantize with the scale from amax, whose
clear and finalize are kernels too, large-tile GEMM) and the SwiGLU-quantize
epilogue are captured once and replayed several times, with eager work
between the replays; every replay must give the eager bytes.  The library
enqueues only kernels (no memset, copy or allocation), so nothing in it is
unsafe to capture."""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_05_amd as nv
from tests.gpu_util import need_gpu
from workloads import activations, normal_weights

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    dev = need_gpu()
    print("[graph] decode 4x12288x5120, prefill 4096x4096x1024, swiglu 512x256x512", flush=True)
    xd = activations("t3_outlier1pct", 4, 5120, seed=11, device=dev)
    wd = nv.quantize(normal_weights(12288, 5120, 0.02, seed=12, device=dev))
    gd = nv.quantize(xd)[2].clone()                                   # calibrated once
    xp = activations("t3_outlier1pct", 4096, 1024, seed=13, device=dev)
    wp = nv.quantize(normal_weights(4096, 1024, 0.02, seed=14, device=dev))   # 256 tiles: large-tile kernel
    xs = activations("t3_outlier1pct", 512, 512, seed=15, device=dev)
    a_s = nv.quantize(xs)
    ws = nv.quantize(normal_weights(512, 512, 0.02, seed=16, device=dev))
    h_gs = torch.tensor([0.01], device=dev)
    out = dict(dc=torch.empty((4, 2560), dtype=torch.uint8, device=dev),
               ds=torch.empty((4, 320), dtype=torch.uint8, device=dev),
               dy=torch.empty((4, 12288), dtype=torch.bfloat16, device=dev),
               pc=torch.empty((4096, 512), dtype=torch.uint8, device=dev),
               ps=torch.empty((4096, 64), dtype=torch.uint8, device=dev),
               pg=torch.empty(1, dtype=torch.float32, device=dev),
               py=torch.empty((4096, 4096), dtype=torch.float32, device=dev),
               sc=torch.empty((512, 128), dtype=torch.uint8, device=dev),
               ss=torch.empty((512, 16), dtype=torch.uint8, device=dev))

    def step():
        nv.quantize(xd, gd, from_amax=False, codes=out["dc"], scales=out["ds"])
        nv.gemm(out["dc"], out["ds"], gd, *wd, out_dtype=torch.bfloat16, out=out["dy"])
        nv.quantize(xp, out["pg"], from_amax=True, codes=out["pc"], scales=out["ps"])
        nv.gemm(out["pc"], out["ps"], out["pg"], *wp, out=out["py"])
        nv.gemm_swiglu_quantize(*a_s, *ws, h_gs, codes=out["sc"], scales=out["ss"])

    step()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in out.items()}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(4):
        for v in out.values():                      # eager work between replays
            v.zero_()
        _ = (xp.float() * 2).sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in out.items():
            assert torch.equal(v, eager[k]), f"replay {r}: {k} differs from the eager result"
    assert float(out["pg"].item()) > 0 and np.isfinite(float(out["pg"].item()))
