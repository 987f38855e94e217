"""GPU quantizer parity: codes, block scales and tensor scales bit-exact
against the CPU oracle (and the hand-worked fixtures)."""
import json
import os

import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_05_amd as nv
from oracle import nvfp4_ref as ref
from tests.gpu_util import assert_codes_equal, gpu_f32, host_f32, need_gpu, oracle_quantize
from workloads import CONFIGS, activations

pytestmark = pytest.mark.gpu


def _gq(x, g=None):
    """GPU quantize; g=None -> tensor scale from amax."""
    if g is None:
        c, s, gs = nv.quantize(x)
    else:
        c, s, gs = nv.quantize(x, gpu_f32(g))
    torch.cuda.synchronize()
    return c, s, gs


def test_hand_worked_blocks(golden_dir):
    need_gpu()
    blocks = json.load(open(os.path.join(golden_dir, "hand_blocks.json")))["blocks"]
    for blk in blocks:
        x = torch.tensor([blk["x"]], dtype=torch.float32).cuda()
        c, s, gs = _gq(x, blk["g"])
        if "g_expected_hex" in blk:
            assert int(np.float32(gs.item()).view(np.uint32)) == int(blk["g_expected_hex"][:8], 16)
            continue
        assert int(s[0, 0]) == int(blk["scale"], 16), blk["name"]
        assert bytes(c[0].cpu().numpy()).hex().upper() == blk["packed"], blk["name"]


def test_every_scale_and_code_round_trips():
    need_gpu()
    rows = []
    for s in range(1, 0x7F):
        vs = ref.E4M3_VALUES[s]
        for m in range(16):
            r = np.zeros(16)
            r[0] = 6.0 * vs
            r[1] = -0.0 if m == 8 else ref.e2m1_decode([m])[0] * vs
            rows.append(r)
    x = np.array(rows, dtype=np.float32)
    c, s, _ = _gq(torch.from_numpy(x).cuda(), 1.0)
    wc, ws, _ = ref.quantize(x, g=1.0)
    assert_codes_equal(c, s, wc, ws, "scale x code brute force")


def test_every_bf16_pattern_beside_fixed_max():
    need_gpu()
    pats = np.arange(0, 1 << 16, dtype=np.uint32)
    vals = (pats << 16).view(np.float32)
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= 96.0)]
    x = np.zeros((vals.size, 16), np.float32)
    x[:, 0] = 96.0
    x[:, 1] = vals
    x[:, 2] = -vals
    xt = torch.from_numpy(x).to(torch.bfloat16).cuda()
    for g in (1.0, 0.0371, 3.3e-3):
        c, s, _ = _gq(xt, g)
        wc, ws, _ = ref.quantize(x, g=g)
        assert_codes_equal(c, s, wc, ws, f"bf16 patterns g={g}")


def _near_tie_rows():
    rows, gs = [], []
    for g in (np.float32(1.0), np.float32(0.3), np.float32(1.7e-3), np.float32(2.9e-5)):
        for s in list(range(1, 0x7F, 3)) + [0x7E]:
            unit = ref.E4M3_VALUES[s] * np.float64(g)
            row = [np.float32(6 * unit)]
            for mid in ref.E2M1_MIDPOINTS:
                t = np.float32(mid * unit)
                row += [t, np.nextafter(t, np.float32(0)), np.nextafter(t, np.float32(1e30))]
            row = np.array(row[:16] + [0.0] * (16 - len(row[:16])), np.float32)
            rows.append(row)
            vals2 = ([np.float32(6 * unit)] + [np.float32(m * unit) for m in ref.E2M1_MIDPOINTS[::-1]]
                     + [np.nextafter(np.float32(m * unit), np.float32(-1)) for m in ref.E2M1_MIDPOINTS])
            rows.append(-np.array(vals2[:16] + [0.0] * (16 - len(vals2[:16])), np.float32))
            gs += [g, g]
    return rows, gs


def test_near_ties_of_codes():
    need_gpu()
    rows, gs = _near_tie_rows()
    for g in sorted(set(gs)):
        x = np.array([r for r, gg in zip(rows, gs) if gg == g], np.float32)
        c, s, _ = _gq(torch.from_numpy(x).cuda(), float(g))
        wc, ws, _ = ref.quantize(x, g=g)
        assert_codes_equal(c, s, wc, ws, f"E2M1 near ties g={g}")


def test_near_ties_of_scales():
    need_gpu()
    for g in (np.float32(1.0), np.float32(0.37), np.float32(3.1e-4), np.float32(7.77e3)):
        rows = []
        for mid in ref.E4M3_MIDPOINTS:
            t = np.float32(mid * 6.0 * np.float64(g))
            for v in (t, np.nextafter(t, np.float32(0)), np.nextafter(t, np.float32(1e38))):
                r = np.zeros(16, np.float32)
                r[5] = v
                r[6] = -v / np.float32(3)
                rows.append(r)
        x = np.array(rows, np.float32)
        c, s, _ = _gq(torch.from_numpy(x).cuda(), float(g))
        wc, ws, _ = ref.quantize(x, g=g)
        assert_codes_equal(c, s, wc, ws, f"E4M3 near ties g={g}")


def bf16_tie_blocks(g):
    """16-value blocks of bf16-exact values on and next to the rounding
    midpoints, for a power-of-two tensor scale g: per block scale s, a block
    maximum 6 val(s) g (scale quotient exactly val(s)), the unit val(s) g, the
    E2M1 midpoints times that unit, and their bf16 neighbours; then blocks whose
    maximum sits on, or next to, an E4M3 midpoint times 6 g.  bf16 data
    reaches exact ties this way (short mantissas), unlike random fp32."""
    def bf16_step(v, d):
        b = np.array([v], np.float32).view(np.uint32)[0] >> 16
        return np.array([(int(b) + d) << 16], np.uint32).view(np.float32)[0]
    blocks = []
    for s in list(range(8, 0x7F, 5)) + [0x7E]:
        unit = np.float32(ref.E4M3_VALUES[s] * np.float64(g))
        mids = [np.float32(m * unit) for m in ref.E2M1_MIDPOINTS]
        blocks.append([np.float32(6 * unit), unit] + mids + [bf16_step(m, -1) for m in mids[:4]]
                      + [bf16_step(m, 1) for m in mids[4:]])
        blocks.append([-np.float32(6 * unit), -unit] + [bf16_step(m, 1) for m in mids] + [-m for m in mids[:4]]
                      + [bf16_step(-m, 1) for m in mids[4:]])
    for mid in ref.E4M3_MIDPOINTS[::4]:
        t = np.float32(mid * 6.0 * np.float64(g))
        for v in (t, bf16_step(t, -1), bf16_step(t, 1)):
            r = [np.float32(0)] * 16
            r[3] = v
            r[9] = -v / np.float32(4)
            blocks.append(r)
    x = np.array(blocks, np.float32)
    assert np.array_equal(torch.from_numpy(x).to(torch.bfloat16).float().numpy(), x)  # exact in bf16
    return x


def test_exact_ties_in_bf16_input():
    need_gpu()
    for g in (np.float32(1.0), np.float32(2.0 ** -7), np.float32(0.5)):
        x = bf16_tie_blocks(g)
        c, s, _ = _gq(torch.from_numpy(x).to(torch.bfloat16).cuda(), float(g))
        wc, ws, _ = ref.quantize(x, g=g)
        assert_codes_equal(c, s, wc, ws, f"bf16 exact ties g={g}")


def test_tensor_scale_from_amax_many_magnitudes():
    need_gpu()
    gen = torch.Generator().manual_seed(3)
    for i in range(40):
        mag = float(10.0 ** (torch.rand(1, generator=gen).item() * 20 - 10))
        x = (torch.randn(8, 64, generator=gen) * mag).to(torch.float32)
        c, s, gs = _gq(x.cuda())
        wc, ws, wg = oracle_quantize(x)
        assert np.float32(gs.item()).view(np.uint32) == np.float32(wg).view(np.uint32), mag
        assert_codes_equal(c, s, wc, ws, f"amax case {i}")


def test_all_zero_tensor_and_zero_blocks():
    need_gpu()
    x = torch.zeros(4, 64, dtype=torch.bfloat16).cuda()
    c, s, gs = _gq(x)
    assert gs.item() == 1.0
    assert int(c.abs().sum()) == 0 and int(s.sum()) == 0
    y = torch.zeros(4, 64)
    y[1, 17] = -3.0
    y[2, :16] = -0.0
    c, s, gs = _gq(y.cuda())
    wc, ws, _ = oracle_quantize(y)
    assert_codes_equal(c, s, wc, ws, "zero blocks and -0.0")


def test_row_stride_and_ragged_rows():
    need_gpu()
    base = activations("t3_outlier1pct", 37, 320, seed=11, device="cpu")
    wide = torch.zeros(37, 384, dtype=torch.bfloat16)
    wide[:, :320] = base
    view = wide.cuda()[:, :320]
    assert view.stride(0) == 384
    c, s, gs = nv.quantize(view)
    torch.cuda.synchronize()
    wc, ws, wg = oracle_quantize(base)
    assert gs.item() == float(wg)
    assert_codes_equal(c, s, wc, ws, "strided rows")


def test_deterministic_repeat():
    need_gpu()
    x = activations("t3_outlier1pct", 256, 5120, seed=5, device="cuda")
    c1, s1, g1 = _gq(x)
    c2, s2, g2 = _gq(x)
    assert torch.equal(c1, c2) and torch.equal(s1, s2) and torch.equal(g1, g2)


@pytest.mark.parametrize("name", ["tiny", "decode", "fused_gdn"])
def test_config_activations_full(name):
    """Every code and scale of the small and medium configs' activations."""
    need_gpu()
    cfg = CONFIGS[name]
    kind, rows, cols, dtype = cfg["x"]
    row_list = cfg.get("ms", (rows,))
    for r in row_list:
        print(f"[quantize parity] {name} rows={r} cols={cols}", flush=True)
        x = activations(kind, r, cols, seed=cfg["seed"], device="cpu", dtype=dtype)
        c, s, gs = _gq(x.cuda())
        wc, ws, wg = oracle_quantize(x)
        assert gs.item() == float(wg)
        assert_codes_equal(c, s, wc, ws, f"{name} rows={r}")


@pytest.mark.parametrize("name", ["tiny", "decode", "fused_gdn"])
def test_config_weights_full(name):
    """Weights are quantized by the same kernel (offline in the pages' recipe)."""
    need_gpu()
    from workloads import normal_weights
    cfg = CONFIGS[name]
    for i, p in enumerate(cfg["projections"]):
        print(f"[quantize parity] {name} weight {p.name} [{p.n}x{p.k}]", flush=True)
        w = normal_weights(p.n, p.k, p.std, seed=cfg["seed"] * 100 + i, device="cpu")
        c, s, gs = _gq(w.cuda())
        wc, ws, wg = ref.quantize(w.numpy())
        assert gs.item() == float(wg)
        assert_codes_equal(c, s, wc, ws, f"{name} weight {p.name}")


def test_zero_rows():
    """No rows: nothing is encoded; the amax mode still writes the tensor scale
    of an all-zero input, 1.0 (the oracle's value for a tensor with no values)."""
    dev = need_gpu()
    print("[quantize] zero rows", flush=True)
    for dtype in (torch.bfloat16, torch.float32):
        x = torch.empty((0, 256), dtype=dtype, device=dev)
        g = torch.full((1,), float("nan"), dtype=torch.float32, device=dev)
        c, s, g = nv.quantize(x, g, from_amax=True)
        torch.cuda.synchronize()
        assert c.shape == (0, 128) and s.shape == (0, 16)
        assert float(g.item()) == float(ref.global_scale(np.zeros((0, 256), np.float32))) == 1.0
        c, s, g2 = nv.quantize(x, torch.tensor([0.5], device=dev), from_amax=False)
        torch.cuda.synchronize()
        assert float(g2.item()) == 0.5
