"""Fused-projection harmonization on the GPU against the oracle, and the
comparison of the fused GDN in-projection: naive fused (one module's scale
for every column), harmonized fused, segmented epilogue (each module's scale
on its columns) and per-module."""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_05_amd as nv
from oracle import nvfp4_ref as ref
from tests.gpu_util import assert_gemm_close, gpu_u8, host_f32, need_gpu
from workloads import CONFIGS, activations, normal_weights

pytestmark = pytest.mark.gpu


def _modules(mults=(1.0, 1.0, 1.0, 1.0), k=None):
    cfg = CONFIGS["fused_gdn"]
    out = []
    for i, (p, mlt) in enumerate(zip(cfg["projections"], mults)):
        w = normal_weights(p.n, k or p.k, p.std, seed=cfg["seed"] * 100 + i, device="cpu") * mlt
        out.append((p.name, ref.quantize(w.numpy())))
    return out


def _gpu_harmonize(mods, k):
    scales = gpu_u8(np.concatenate([q[1] for _, q in mods]))
    gs = torch.tensor([float(q[2]) for _, q in mods], dtype=torch.float32, device="cuda")
    rows = [q[0].shape[0] for _, q in mods]
    shared, counters = nv.harmonize_fused_scales(scales, gs, rows, k)
    torch.cuda.synchronize()
    return scales.cpu().numpy(), float(shared.item()), counters.cpu().numpy().astype(np.int64)


@pytest.mark.parametrize("mults", [(1.0, 1.0, 1.0, 1.0), (1.0, 1.0, 4.0, 0.25), (1.0, 3.7, 0.011, 250.0)])
def test_harmonize_matches_oracle(mults):
    need_gpu()
    mods = _modules(mults, k=1024)
    got, g_star, counters = _gpu_harmonize(mods, 1024)
    want, w_star, n_inexact, n_sub = ref.harmonize_ref([q[1] for _, q in mods], [q[2] for _, q in mods])
    assert g_star == float(w_star)
    assert np.array_equal(got, want)
    assert counters[0] == n_inexact and counters[1] == n_sub


def test_harmonize_power_of_two_ratios_exact():
    need_gpu()
    mods = _modules(k=512)
    base = mods[0][1][2]
    mods = [(n, (c, s, np.float32(base * f))) for (n, (c, s, _)), f in zip(mods, (1.0, 0.5, 0.125, 2.0))]
    got, g_star, counters = _gpu_harmonize(mods, 512)
    assert g_star == float(np.float32(base * 2.0))
    assert counters[0] == 0 and counters[1] == 0
    want, _, _, _ = ref.harmonize_ref([q[1] for _, q in mods], [q[2] for _, q in mods])
    assert np.array_equal(got, want)


def _harmonize_bytes(scales_np, gs, rows, k, offset=0):
    """GPU harmonize of a flat byte buffer placed `offset` bytes into its
    allocation (offset 1: a misaligned buffer, taken byte by byte)."""
    buf = torch.zeros(scales_np.size + 16, dtype=torch.uint8, device="cuda")
    view = buf[offset:offset + scales_np.size]
    view.copy_(torch.from_numpy(np.ascontiguousarray(scales_np).reshape(-1)))
    shared, counters = nv.harmonize_fused_scales(view, torch.tensor(gs, dtype=torch.float32, device="cuda"),
                                                 rows, k)
    torch.cuda.synchronize()
    out = buf.cpu().numpy()
    assert not out[:offset].any() and not out[offset + scales_np.size:].any(), "wrote outside the buffer"
    return out[offset:offset + scales_np.size], float(shared.item()), counters.cpu().numpy().astype(np.int64)


@pytest.mark.parametrize("offset", [0, 1])
def test_harmonize_every_scale_byte_of_every_module(offset):
    # one row per module holding every E4M3 scale byte 0x00..0x7E, so every
    # (scale, module) pair of the kernel's lookup table is checked
    need_gpu()
    gs = [np.float32(v) for v in (0.0123, 0.5, 3.7e-3, 1.0, 7.25e-5)]
    rows = [1] * len(gs)
    k = 16 * 127
    mods = [np.arange(127, dtype=np.uint8).reshape(1, 127) for _ in gs]
    got, g_star, counters = _harmonize_bytes(np.concatenate(mods), gs, rows, k, offset)
    want, w_star, n_inexact, n_sub = ref.harmonize_ref(mods, gs)
    assert g_star == float(w_star)
    assert np.array_equal(got, want.reshape(-1))
    assert counters[0] == n_inexact and counters[1] == n_sub


@pytest.mark.parametrize("offset", [0, 1])
def test_harmonize_ragged_rows_and_module_ends_inside_chunks(offset):
    # 17 scales per row, so 16-byte chunks straddle rows and module ends; an
    # empty module; random scale bytes
    need_gpu()
    rng = np.random.default_rng(5 + offset)
    rows = [5, 0, 3, 7, 1, 40]
    gs = [np.float32(v) for v in (0.02, 0.3, 0.02, 1.5e-3, 4.0, 0.25)]
    k = 16 * 17
    mods = [rng.integers(0, 0x7F, size=(r, 17)).astype(np.uint8) for r in rows]
    got, g_star, counters = _harmonize_bytes(np.concatenate(mods), gs, rows, k, offset)
    want, w_star, n_inexact, n_sub = ref.harmonize_ref(mods, gs)
    assert g_star == float(w_star)
    assert np.array_equal(got, want.reshape(-1))
    assert counters[0] == n_inexact and counters[1] == n_sub


def test_fused_gdn_fused_variants():
    """C4: naive fused, harmonized fused and segmented epilogue against their
    oracles on every output element (4096 tokens x 12384 columns), and
    harmonized against per-module."""
    need_gpu()
    cfg = CONFIGS["fused_gdn"]
    kind, rows, cols, dtype = cfg["x"]
    x = activations(kind, rows, cols, seed=cfg["seed"], device="cpu", dtype=dtype)
    for mults in ((1.0, 1.0, 1.0, 1.0), (1.0, 1.0, 4.0, 0.25)):
        print(f"[fused gdn] module multipliers {mults}", flush=True)
        mods = _modules(mults)
        ac, as_, ga = nv.quantize(x.cuda())                   # GPU activations
        oa = ref.quantize(host_f32(x))                        # oracle activations (bit-equal)
        assert np.array_equal(ac.cpu().numpy(), oa[0]) and np.array_equal(as_.cpu().numpy(), oa[1])
        wc = np.concatenate([q[0] for _, q in mods])
        ws = np.concatenate([q[1] for _, q in mods])
        gs = [q[2] for _, q in mods]
        gs_dev = torch.tensor([float(g) for g in gs], dtype=torch.float32, device="cuda")

        naive = nv.gemm(ac, as_, ga, gpu_u8(wc), gpu_u8(ws), gs_dev[0:1])
        ws_dev = gpu_u8(ws)
        shared, _ = nv.harmonize_fused_scales(ws_dev, gs_dev, [q[0].shape[0] for _, q in mods], cols)
        harm = nv.gemm(ac, as_, ga, gpu_u8(wc), ws_dev, shared)
        seg = nv.gemm_segmented(ac, as_, ga, gpu_u8(wc), gpu_u8(ws), gs_dev, [q[0].shape[0] for _, q in mods])
        torch.cuda.synchronize()

        # every output element of the 4096 x 12384 results against the fp64 oracle
        a_s = oa
        Yn, Sn = ref.naive_fused_ref(*a_s, wc, ws, gs)
        assert_gemm_close(naive, Yn, Sn, "naive fused")
        del Yn, Sn
        Ys, Ss = ref.gemm_segmented_ref(*a_s, wc, ws, gs, [q[0].shape[0] for _, q in mods])
        assert_gemm_close(seg, Ys, Ss, "segmented epilogue")
        del Ys, Ss
        hs, hg, _, _ = ref.harmonize_ref([q[1] for _, q in mods], gs)
        assert np.array_equal(ws_dev.cpu().numpy(), hs) and float(shared.item()) == float(hg)
        Yh, Sh = ref.gemm_ref(*a_s, wc, hs, hg)
        assert_gemm_close(harm, Yh, Sh, "harmonized fused")
        del Yh, Sh
        # harmonized vs the per-module result: only E4M3 re-rounding separates them
        row = 0
        harm_h = harm.cpu().numpy().astype(np.float64)
        for name, (c, s, g) in mods:
            Yp, Sp = ref.gemm_ref(*a_s, c, s, g)
            block = harm_h[:, row:row + c.shape[0]]
            rel = np.linalg.norm(block - Yp) / max(np.linalg.norm(Yp), 1e-300)
            print(f"  {name}: harmonized vs per-module relative error {rel:.3e}; "
                  f"naive/per-module scale ratio {float(gs[0]) / float(g):.4f}", flush=True)
            assert rel < 2.0 ** -4
            row += c.shape[0]
