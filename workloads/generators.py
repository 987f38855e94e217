"""Seeded input recipes for the five workloads of the NVFP4 linear-layer path.

The value distributions follow what the pages report for the residual
stream that feeds the projections: the anthology record LIT-800 ("Key
takeaways", block-scaling bullet, i.e. the paper's section 5.1 / Table 2)
gives a median-layer max/RMS of 63.5, a kurtosis near 1,560 and outliers of
48-368x the RMS.  The captured activations themselves are not available, so
these generators stand in for them.  Shapes are those of a ~27B hybrid
Gated-DeltaNet model: hidden 5120, GDN qkv 8192 / z 4096 / a 48 / b 48,
GDN out-projection input 4096, MLP intermediate 17408.

All draws use ``torch.Generator`` seeded per tensor; ``device`` selects
where the values are made (the CPU for oracle-sized cases, the GPU for the
full-size ones, whose sampled rows are then copied back for the oracle).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

HIDDEN = 5120
# Magnitude of the lognormal workload's outlier channel: with one constant
# channel of magnitude R among C = 5120 unit-RMS ones the kurtosis is about
# R^4 / (C (1 + R^2 / C)^2), ~1.5e3 at R = 76, the level the pages report
# for the median layer (LIT-800, "Key takeaways", block-scaling bullet).
OUTLIER_MAGNITUDE = 76.0


@dataclass(frozen=True)
class ProjectionSpec:
    name: str
    n: int        # output features
    k: int        # input features
    std: float    # weight init standard deviation


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _student_t3(shape, gen, device):
    """Student-t with 3 degrees of freedom: Z / sqrt(chi2_3 / 3)."""
    z = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    chi = torch.zeros(shape, device=device, dtype=torch.float32)
    for _ in range(3):
        e = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        chi.add_(e * e)
    return z / torch.sqrt(chi / 3.0)


def activations(kind: str, rows: int, cols: int, seed: int, device="cpu",
                dtype=torch.bfloat16, row_chunk: int = 4096) -> torch.Tensor:
    """Activation matrix [rows, cols].

    kind:
      "gauss_outlier2"  N(0,1) with 2 random channels scaled x50
      "t3_outlier1pct"  Student-t(3) with 1% of channels scaled x60
      "lognormal_rms"   per-channel RMS exp(1.5 z) times N(0,1), plus one
                        outlier channel of constant magnitude 76 (random
                        sign) against the base tensor RMS of 1: kurtosis
                        ~1.4e3-1.5e3 and max/RMS ~50-65 at widths 4096 and
                        5120; at width 17408 the largest lognormal channel
                        (more channels, a longer tail) sets max/RMS ~127
    Rows are drawn in chunks from one seeded stream so large tensors never
    need a second full-size temporary.
    """
    gen = _gen(seed, device)
    out = torch.empty((rows, cols), device=device, dtype=dtype)
    cgen = _gen(seed + 7919, "cpu")  # channel choices on the host: same on any device
    if kind == "gauss_outlier2":
        ch = torch.randperm(cols, generator=cgen)[:2]
        mult = torch.ones(cols)
        mult[ch] = 50.0
    elif kind == "t3_outlier1pct":
        ch = torch.randperm(cols, generator=cgen)[: max(1, cols // 100)]
        mult = torch.ones(cols)
        mult[ch] = 60.0
    elif kind == "lognormal_rms":
        rms = torch.exp(1.5 * torch.randn(cols, generator=cgen))
        rms = rms / torch.sqrt(torch.mean(rms * rms))          # tensor RMS 1
        ch = torch.randperm(cols, generator=cgen)[:1]
        mult = rms
    else:
        raise ValueError(f"unknown activation kind {kind!r}")
    mult = mult.to(device=device, dtype=torch.float32)
    for r0 in range(0, rows, row_chunk):
        r1 = min(rows, r0 + row_chunk)
        if kind == "t3_outlier1pct":
            v = _student_t3((r1 - r0, cols), gen, device)
        else:
            v = torch.randn((r1 - r0, cols), generator=gen, device=device, dtype=torch.float32)
        v = v * mult
        if kind == "lognormal_rms":
            # a "massive activation" channel: constant magnitude, random sign
            v[:, ch.to(device)] = OUTLIER_MAGNITUDE * torch.sign(v[:, ch.to(device)])
        out[r0:r1] = v.to(dtype)
    return out


def normal_weights(n: int, k: int, std: float, seed: int, device="cpu",
                   row_chunk: int = 4096) -> torch.Tensor:
    """Weight matrix [n, k] (out x in, K contiguous) drawn from N(0, std^2), fp32."""
    gen = _gen(seed, device)
    out = torch.empty((n, k), device=device, dtype=torch.float32)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        out[r0:r1] = torch.randn((r1 - r0, k), generator=gen, device=device) * std
    return out


def stats(x: torch.Tensor, max_rows: int = 4096) -> dict:
    """max/RMS and kurtosis of (a row sample of) a tensor, reported beside results."""
    xs = x[:max_rows].double().flatten()
    rms = float(torch.sqrt(torch.mean(xs * xs)))
    m2 = float(torch.mean(xs * xs))
    m4 = float(torch.mean(xs ** 4))
    return {"max_over_rms": float(xs.abs().max()) / rms if rms > 0 else 0.0,
            "kurtosis": m4 / (m2 * m2) if m2 > 0 else 0.0}


# Workloads: one entry per configuration, with its projections.
CONFIGS = {
    "tiny": {
        "desc": "X[16x256] fp32 N(0,1) with 2 outlier channels x50; W[256x256] N(0,0.02); seed 0",
        "x": ("gauss_outlier2", 16, 256, torch.float32),
        "projections": [ProjectionSpec("w", 256, 256, 0.02)],
        "seed": 0,
    },
    "decode": {
        "desc": "X[M x 5120] bf16 Student-t(3) with 1% channels x60, M in {1,8,32,64}; "
                "fused GDN in-projection W[12288x5120] N(0,0.02); seed 1",
        "ms": (1, 8, 32, 64),
        "x": ("t3_outlier1pct", None, HIDDEN, torch.bfloat16),
        "projections": [ProjectionSpec("in_proj", 12288, HIDDEN, 0.02)],
        "seed": 1,
    },
    "prefill_mlp": {
        "desc": "X[32768x5120] and X_d[32768x17408] bf16 Student-t(3) with 1% channels x60; "
                "W_gu[34816x5120] and W_d[5120x17408] N(0,0.015); seed 2",
        "rows": 32768,
        "x": ("t3_outlier1pct", 32768, HIDDEN, torch.bfloat16),
        "projections": [ProjectionSpec("gate_up", 34816, HIDDEN, 0.015),
                        ProjectionSpec("down", HIDDEN, 17408, 0.015)],
        "seed": 2,
    },
    "fused_gdn": {
        "desc": "X[4096x5120] bf16 Student-t(3) with 1% channels x60; qkv[8192], z[4096], "
                "a[48], b[48] x 5120 N(0,0.02), each with its own tensor scale; seed 3",
        "rows": 4096,
        "x": ("t3_outlier1pct", 4096, HIDDEN, torch.bfloat16),
        "projections": [ProjectionSpec("qkv", 8192, HIDDEN, 0.02),
                        ProjectionSpec("z", 4096, HIDDEN, 0.02),
                        ProjectionSpec("a", 48, HIDDEN, 0.02),
                        ProjectionSpec("b", 48, HIDDEN, 0.02)],
        "seed": 3,
    },
    "layer_32k": {
        "desc": "one hybrid layer at 32768 tokens: GDN qkv/z/a/b fused in-projection "
                "[12384x5120], out [5120x4096], MLP gate/up [34816x5120], down [5120x17408]; "
                "inputs [32768 x {5120,4096,17408}] bf16 with lognormal per-channel RMS "
                "(sigma 1.5) and one constant-magnitude 76x outlier channel; seed 4",
        "rows": 32768,
        "x": ("lognormal_rms", 32768, HIDDEN, torch.bfloat16),
        "projections": [ProjectionSpec("qkv", 8192, HIDDEN, 0.02),
                        ProjectionSpec("z", 4096, HIDDEN, 0.02),
                        ProjectionSpec("a", 48, HIDDEN, 0.02),
                        ProjectionSpec("b", 48, HIDDEN, 0.02),
                        ProjectionSpec("out", HIDDEN, 4096, 0.02),
                        ProjectionSpec("gate_up", 34816, HIDDEN, 0.015),
                        ProjectionSpec("down", HIDDEN, 17408, 0.015)],
        "seed": 4,
    },
}


def gemm_flops(m: int, n: int, k: int) -> float:
    return 2.0 * m * n * k


__all__ = ["CONFIGS", "ProjectionSpec", "activations", "normal_weights", "stats",
           "gemm_flops", "HIDDEN"]
