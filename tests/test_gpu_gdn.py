"""nvfp4_gdn_recurrence against the fp64 recurrence reference.

Tolerance (from the arithmetic, as the header states): a token's fp32
rounding adds at most (128 + 16) 2^-24 M_t to the state error, with M_t the
running maximum over s <= t of |S_s|_F + beta_s |v_s|, and the update carries
the earlier error through its linear part alpha I - beta khat khat^T, whose
spectral norm c_t = max(alpha_t, |alpha_t - beta_t|) is at most 1:
e_t <= c_t e_{t-1} + (128 + 16) 2^-24 M_t, which never exceeds
t (128 + 16) 2^-24 M_t.  An output o_t = S_t^T qhat / sqrt(128) then differs
by at most (e_t + 128 2^-24 |S_t|_F) / sqrt(128)."""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_05_amd as nv
from oracle import gdn_ref as G
from tests.gpu_util import need_gpu

pytestmark = pytest.mark.gpu
D = 128
LAYOUT = dict(q_col=0, k_col=2 * D, v_col=4 * D, g_col=8 * D, beta_col=8 * D + 4)  # n_qk 2, n_v 4
LDX = 8 * D + 16


def _rows(T, seed, v_zero=False):
    """Projection rows: q, k, v ~ N(0, 1); g = -exp(A_log) softplus(a + dt_bias)
    with A = U(1, 16), dt_bias for dt in [1e-3, 0.1], a ~ N(0, 1); beta = sigmoid(N(0, 1))."""
    rng = np.random.default_rng(seed)
    x = np.zeros((T, LDX), np.float32)
    x[:, :8 * D] = rng.standard_normal((T, 8 * D))
    if v_zero:
        x[:, 4 * D:8 * D] = 0
    a_log = np.log(rng.uniform(1, 16, 4))
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), 4))
    dt_bias = dt + np.log(-np.expm1(-dt))
    z = rng.standard_normal((T, 4)) + dt_bias
    x[:, 8 * D:8 * D + 4] = -np.exp(a_log) * (np.maximum(z, 0) + np.log1p(np.exp(-np.abs(z))))
    x[:, 8 * D + 4:8 * D + 8] = 1 / (1 + np.exp(-rng.standard_normal((T, 4))))
    return x


def _contraction_bound(g, beta, M):
    """Error allowance of the fp32 state that uses the update's contraction:
    the linear part of S -> alpha S + beta k (v - S^T k)^T is alpha I - beta k k^T
    (|k| = 1), whose spectral norm is c = max(alpha, |alpha - beta|) <= 1, so
    e_t <= c_t e_{t-1} + (D + 16) 2^-24 M_t (the per-token rounding term above)."""
    alpha = np.exp(np.asarray(g, np.float64))
    c = np.maximum(alpha, np.abs(alpha - beta))
    d = (D + 16) * 2.0 ** -24 * M
    e, acc = np.empty_like(d), np.zeros(d.shape[1])
    for t in range(d.shape[0]):
        acc = c[t] * acc + d[t]
        e[t] = acc
    return e


def _check(x, s0=None, snaps=(), v_col=4 * D):
    dev = need_gpu()
    T = x.shape[0]
    lay = dict(LAYOUT, v_col=v_col)
    xt = torch.from_numpy(x).to(dev)
    so = torch.empty((4, D, D), dtype=torch.float32, device=dev)
    o = torch.full((T, 4 * D + 32), np.nan, dtype=torch.float32, device=dev)   # ldo > 4 D
    nr = torch.empty((T, 4), dtype=torch.float32, device=dev)
    st = torch.tensor(list(snaps), dtype=torch.int32, device=dev) if snaps else None
    sn = torch.empty((len(snaps), 4, D, D), dtype=torch.float32, device=dev) if snaps else None
    nv.gdn_recurrence(xt, **lay, n_qk_heads=2, n_v_heads=4,
                      state_in=None if s0 is None else torch.from_numpy(s0.astype(np.float32)).to(dev),
                      state_out=so, o=o, state_norms=nr, snap_steps=st, snaps=sn)
    torch.cuda.synchronize()
    q, k, v, g, beta = G.split_projection_rows(x, **lay, n_qk=2, n_v=4)
    O, S, SN, NR = G.gdn_recurrence_ref(q, k, v, g, beta, s0=s0, snap_steps=snaps)
    # running bound M_t per head and the per-token error allowance
    norm_S = np.sqrt(NR)                                         # [T, heads]
    drive = beta * np.linalg.norm(v, axis=2)
    M = np.maximum.accumulate(norm_S + drive, axis=0)
    if s0 is not None:
        M = np.maximum(M, np.linalg.norm(s0.reshape(4, -1), axis=1)[None, :])
    e_S = _contraction_bound(g, beta, M)                          # [T, heads]
    # final state
    err = np.linalg.norm((so.cpu().numpy() - S).reshape(4, -1), axis=1)
    assert np.all(err <= e_S[-1]), f"state error {err} > {e_S[-1]}"
    # outputs, per token and head
    ov = o.cpu().numpy()
    assert np.all(np.isnan(ov[:, 4 * D:])), "o written past its columns"
    oe = np.linalg.norm(ov[:, :4 * D].reshape(T, 4, D) - O, axis=2)
    o_tol = (e_S + D * 2.0 ** -24 * norm_S) / np.sqrt(D)
    assert np.all(oe <= o_tol), f"output error {oe.max()} (worst ratio {np.max(oe / o_tol):.3f})"
    # norms and snapshots
    assert np.all(np.abs(np.sqrt(nr.cpu().numpy()) - norm_S) <= e_S + 1e-30)
    for i, s in enumerate(snaps):
        se = np.linalg.norm((sn[i].cpu().numpy() - SN[i]).reshape(4, -1), axis=1)
        assert np.all(se <= e_S[s]), f"snapshot {s}: {se} > {e_S[s]}"
    return float(np.max(err / e_S[-1]))


def test_recurrence_short_with_snapshots():
    print("[gdn] T=300 snapshots", flush=True)
    _check(_rows(300, 1), snaps=(0, 1, 77, 150, 299))


def test_recurrence_from_a_start_state():
    print("[gdn] T=257 start state", flush=True)
    rng = np.random.default_rng(7)
    _check(_rows(257, 2), s0=rng.standard_normal((4, D, D)) * 0.05, snaps=(3, 256))


def test_recurrence_carries_a_perturbation_with_zero_v():
    # v_col = -1: the state is a perturbation; it decays by the same operator
    print("[gdn] T=200 v = 0, impulse", flush=True)
    rng = np.random.default_rng(8)
    x = _rows(200, 3, v_zero=True)
    _check(x, s0=rng.standard_normal((4, D, D)) * 0.01, v_col=-1)


def test_recurrence_long():
    print("[gdn] T=3000", flush=True)
    _check(_rows(3000, 4), snaps=(999, 2999))


def test_single_token_and_empty():
    print("[gdn] T=1 and T=0", flush=True)
    _check(_rows(1, 5), snaps=(0,))
    dev = need_gpu()
    nv.gdn_recurrence(torch.zeros((0, LDX), dtype=torch.float32, device=dev), **LAYOUT, n_qk_heads=2, n_v_heads=4)
    # no tokens: S_0 is the start state, or zeros without one
    s0 = torch.randn((4, D, D), dtype=torch.float32, device=dev)
    so = torch.full((4, D, D), np.nan, dtype=torch.float32, device=dev)
    nv.gdn_recurrence(torch.zeros((0, LDX), dtype=torch.float32, device=dev), **LAYOUT, n_qk_heads=2, n_v_heads=4,
                      state_in=s0, state_out=so)
    torch.cuda.synchronize()
    assert torch.equal(so, s0)
    nv.gdn_recurrence(torch.zeros((0, LDX), dtype=torch.float32, device=dev), **LAYOUT, n_qk_heads=2, n_v_heads=4,
                      state_out=so)
    torch.cuda.synchronize()
    assert torch.equal(so, torch.zeros_like(so))


def _check_heads(T, n_qk, n_v, seed):
    """The same checks for another head layout: q | k | v | g | beta packed
    from column 0, with n_qk q/k heads and n_v value heads."""
    dev = need_gpu()
    rng = np.random.default_rng(seed)
    q_col, k_col, v_col = 0, n_qk * D, 2 * n_qk * D
    g_col = v_col + n_v * D
    b_col = g_col + n_v
    x = np.zeros((T, b_col + n_v), np.float32)
    x[:, :g_col] = rng.standard_normal((T, g_col))
    x[:, g_col:b_col] = -np.exp(rng.uniform(0, 2.7, n_v)) * np.log1p(np.exp(rng.standard_normal((T, n_v)) - 4))
    x[:, b_col:] = 1 / (1 + np.exp(-rng.standard_normal((T, n_v))))
    so = torch.empty((n_v, D, D), dtype=torch.float32, device=dev)
    o = torch.empty((T, n_v * D), dtype=torch.float32, device=dev)
    nv.gdn_recurrence(torch.from_numpy(x).to(dev), q_col=q_col, k_col=k_col, v_col=v_col, g_col=g_col,
                      beta_col=b_col, n_qk_heads=n_qk, n_v_heads=n_v, state_out=so, o=o)
    torch.cuda.synchronize()
    q, k, v, g, beta = G.split_projection_rows(x, q_col, k_col, v_col, g_col, b_col, n_qk, n_v)
    O, S, _, NR = G.gdn_recurrence_ref(q, k, v, g, beta)
    M = np.maximum.accumulate(np.sqrt(NR) + beta * np.linalg.norm(v, axis=2), axis=0)
    e_S = _contraction_bound(g, beta, M)
    err = np.linalg.norm((so.cpu().numpy() - S).reshape(n_v, -1), axis=1)
    assert np.all(err <= e_S[-1]), f"state error {err} > {e_S[-1]}"
    oe = np.linalg.norm(o.cpu().numpy().reshape(T, n_v, D) - O, axis=2)
    assert np.all(oe <= (e_S + D * 2.0 ** -24 * np.sqrt(NR)) / np.sqrt(D))


@pytest.mark.parametrize("T,n_qk,n_v", [(6, 2, 2), (7, 1, 4), (130, 3, 3), (203, 2, 8)])
def test_recurrence_head_layouts_and_token_remainders(T, n_qk, n_v):
    # T % 4 = 2, 3, 2, 3: the loop runs in groups of 4 tokens
    print(f"[gdn] T={T} n_qk={n_qk} n_v={n_v}", flush=True)
    _check_heads(T, n_qk, n_v, seed=T)


@pytest.mark.parametrize("want_o,want_norms", [(False, False), (False, True), (True, False), (True, True)])
def test_recurrence_output_combinations(want_o, want_norms):
    # each combination of outputs runs its own kernel variant (q is not read
    # without o; the norms take a whole head per workgroup)
    print(f"[gdn] T=301 o={want_o} norms={want_norms}", flush=True)
    dev = need_gpu()
    x = _rows(301, 11)
    rng = np.random.default_rng(12)
    s0 = rng.standard_normal((4, D, D)) * 0.05
    so = torch.empty((4, D, D), dtype=torch.float32, device=dev)
    o = torch.empty((301, 4 * D), dtype=torch.float32, device=dev) if want_o else None
    nr = torch.empty((301, 4), dtype=torch.float32, device=dev) if want_norms else None
    steps = (0, 63, 64, 200)
    st = torch.tensor(steps, dtype=torch.int32, device=dev)
    sn = torch.empty((len(steps), 4, D, D), dtype=torch.float32, device=dev)
    nv.gdn_recurrence(torch.from_numpy(x).to(dev), **LAYOUT, n_qk_heads=2, n_v_heads=4,
                      state_in=torch.from_numpy(s0.astype(np.float32)).to(dev), state_out=so, o=o,
                      state_norms=nr, snap_steps=st, snaps=sn)
    torch.cuda.synchronize()
    q, k, v, g, beta = G.split_projection_rows(x, **LAYOUT, n_qk=2, n_v=4)
    O, S, SN, NR = G.gdn_recurrence_ref(q, k, v, g, beta, s0=s0, snap_steps=steps)
    norm_S = np.sqrt(NR)
    M = np.maximum.accumulate(norm_S + beta * np.linalg.norm(v, axis=2), axis=0)
    M = np.maximum(M, np.linalg.norm(s0.reshape(4, -1), axis=1)[None, :])
    e_S = _contraction_bound(g, beta, M)
    err = np.linalg.norm((so.cpu().numpy() - S).reshape(4, -1), axis=1)
    assert np.all(err <= e_S[-1]), f"state error {err} > {e_S[-1]}"
    for i, s in enumerate(steps):
        se = np.linalg.norm((sn[i].cpu().numpy() - SN[i]).reshape(4, -1), axis=1)
        assert np.all(se <= e_S[s]), f"snapshot {s}: {se} > {e_S[s]}"
    if want_o:
        oe = np.linalg.norm(o.cpu().numpy().reshape(301, 4, D) - O, axis=2)
        assert np.all(oe <= (e_S + D * 2.0 ** -24 * norm_S) / np.sqrt(D))
    if want_norms:
        assert np.all(np.abs(np.sqrt(nr.cpu().numpy()) - norm_S) <= e_S + 1e-30)


def test_snapshot_steps_out_of_order_or_past_the_end_are_skipped():
    # slot i holds S after step i; a step not above the previous one, or not
    # below T, leaves its slot unwritten
    print("[gdn] T=40 snapshot steps (5, 3, 10, 10, 39, 40)", flush=True)
    dev = need_gpu()
    x = _rows(40, 21)
    steps = (5, 3, 10, 10, 39, 40)
    st = torch.tensor(steps, dtype=torch.int32, device=dev)
    sn = torch.full((len(steps), 4, D, D), np.nan, dtype=torch.float32, device=dev)
    nv.gdn_recurrence(torch.from_numpy(x).to(dev), **LAYOUT, n_qk_heads=2, n_v_heads=4, snap_steps=st, snaps=sn)
    torch.cuda.synchronize()
    q, k, v, g, beta = G.split_projection_rows(x, **LAYOUT, n_qk=2, n_v=4)
    _, _, SN, NR = G.gdn_recurrence_ref(q, k, v, g, beta, snap_steps=(5, 10, 39))
    M = np.maximum.accumulate(np.sqrt(NR) + beta * np.linalg.norm(v, axis=2), axis=0)
    e_S = _contraction_bound(g, beta, M)
    got = sn.cpu().numpy()
    for slot, ref_i, t in ((0, 0, 5), (2, 1, 10), (4, 2, 39)):
        err = np.linalg.norm((got[slot] - SN[ref_i]).reshape(4, -1), axis=1)
        assert np.all(err <= e_S[t]), f"slot {slot} (token {t}): {err} > {e_S[t]}"
    for slot in (1, 3, 5):
        assert np.all(np.isnan(got[slot])), f"slot {slot} was written"


@pytest.mark.parametrize("want_norms", [False, True])
def test_recurrence_many_chunks_and_segments(want_norms):
    # 9000 tokens: 141 chunks of 64 per-token scalars; snapshots inside,
    # at and next to chunk edges restart the ring at unaligned tokens
    print(f"[gdn] T=9000 norms={want_norms}", flush=True)
    dev = need_gpu()
    T = 9000
    x = _rows(T, 31)
    steps = (63, 64, 130, 4095, 8999)
    so = torch.empty((4, D, D), dtype=torch.float32, device=dev)
    o = torch.empty((T, 4 * D), dtype=torch.float32, device=dev)
    nr = torch.empty((T, 4), dtype=torch.float32, device=dev) if want_norms else None
    st = torch.tensor(steps, dtype=torch.int32, device=dev)
    sn = torch.empty((len(steps), 4, D, D), dtype=torch.float32, device=dev)
    nv.gdn_recurrence(torch.from_numpy(x).to(dev), **LAYOUT, n_qk_heads=2, n_v_heads=4, state_out=so, o=o,
                      state_norms=nr, snap_steps=st, snaps=sn)
    torch.cuda.synchronize()
    q, k, v, g, beta = G.split_projection_rows(x, **LAYOUT, n_qk=2, n_v=4)
    O, S, SN, NR = G.gdn_recurrence_ref(q, k, v, g, beta, snap_steps=steps)
    norm_S = np.sqrt(NR)
    M = np.maximum.accumulate(norm_S + beta * np.linalg.norm(v, axis=2), axis=0)
    e_S = _contraction_bound(g, beta, M)
    err = np.linalg.norm((so.cpu().numpy() - S).reshape(4, -1), axis=1)
    assert np.all(err <= e_S[-1]), f"state error {err} > {e_S[-1]}"
    for i, s in enumerate(steps):
        se = np.linalg.norm((sn[i].cpu().numpy() - SN[i]).reshape(4, -1), axis=1)
        assert np.all(se <= e_S[s]), f"snapshot {s}: {se} > {e_S[s]}"
    oe = np.linalg.norm(o.cpu().numpy().reshape(T, 4, D) - O, axis=2)
    assert np.all(oe <= (e_S + D * 2.0 ** -24 * norm_S) / np.sqrt(D))
    if want_norms:
        assert np.all(np.abs(np.sqrt(nr.cpu().numpy()) - norm_S) <= e_S + 1e-30)


def test_recurrence_layer_32k_full_size():
    """The recurrence in the bench's configuration: 32768 tokens, 16 q/k and 32
    value heads of 128 in rows of 12384 values (q | k | v | z | a | b),
    snapshots only; then the impulse form (v = 0, a start state, norms) over
    the second half.  The oracle follows value heads 0 and 31 (q/k heads 0
    and 15); the other heads are checked for finite values."""
    dev = need_gpu()
    T, ldx, n_qk, n_v = 32768, 12384, 16, 32
    g_col, b_col = 12288, 12336
    lay = dict(q_col=0, k_col=2048, v_col=4096, g_col=g_col, beta_col=b_col, n_qk_heads=n_qk, n_v_heads=n_v)
    print(f"[gdn] full size T={T} heads {n_qk}/{n_v} ldx={ldx}", flush=True)
    gen = torch.Generator(device=dev).manual_seed(2024)
    x = torch.randn((T, ldx), generator=gen, device=dev)
    rng = np.random.default_rng(7)
    a_log = torch.from_numpy(np.log(rng.uniform(1, 16, n_v))).float().to(dev)
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), n_v))
    dt_bias = torch.from_numpy(dt + np.log(-np.expm1(-dt))).float().to(dev)
    x[:, g_col:g_col + n_v] = -torch.exp(a_log) * torch.nn.functional.softplus(x[:, g_col:g_col + n_v] + dt_bias)
    x[:, b_col:b_col + n_v] = torch.sigmoid(x[:, b_col:b_col + n_v])
    steps = [255, 1023, 4095, 8191, 16383, 24575, 32767]
    sn = torch.empty((len(steps), n_v, D, D), dtype=torch.float32, device=dev)
    nv.gdn_recurrence(x, **lay, snap_steps=torch.tensor(steps, dtype=torch.int32, device=dev), snaps=sn)
    t0 = T // 2
    s0 = 0.01 * torch.randn((n_v, D, D), generator=gen, device=dev)
    nrm = torch.empty((T - t0, n_v), dtype=torch.float32, device=dev)
    nv.gdn_recurrence(x[t0:], **dict(lay, v_col=-1), state_in=s0, state_norms=nrm)
    torch.cuda.synchronize()
    assert torch.isfinite(sn).all() and torch.isfinite(nrm).all()

    vh = np.array([0, 31])
    qh = vh * n_qk // n_v

    def cols(c0, heads):
        return np.concatenate([c0 + h * D + np.arange(D) for h in heads])

    sel = np.concatenate([cols(0, qh), cols(2048, qh), cols(4096, vh), g_col + vh, b_col + vh])
    xs = x[:, torch.from_numpy(sel).to(dev)].cpu().numpy()
    del x
    q, k, v, g, beta = G.split_projection_rows(xs, q_col=0, k_col=2 * D, v_col=4 * D, g_col=6 * D,
                                               beta_col=6 * D + 2, n_qk=2, n_v=2)
    _, _, SN, NR = G.gdn_recurrence_ref(q, k, v, g, beta, snap_steps=steps)
    M = np.maximum.accumulate(np.sqrt(NR) + beta * np.linalg.norm(v, axis=2), axis=0)
    e = _contraction_bound(g, beta, M)
    worst = 0.0
    for i, s in enumerate(steps):
        se = np.linalg.norm((sn[i][torch.from_numpy(vh).to(dev)].cpu().numpy() - SN[i]).reshape(2, -1), axis=1)
        assert np.all(se <= e[s]), f"snapshot {s}: {se} > {e[s]}"
        worst = max(worst, float(np.max(se / e[s])))
    # impulse form: v = 0 from the start state, norms per token
    s0h = s0[torch.from_numpy(vh).to(dev)].cpu().numpy()
    _, _, _, NR2 = G.gdn_recurrence_ref(q[t0:], k[t0:], np.zeros_like(v[t0:]), g[t0:], beta[t0:], s0=s0h)
    M2 = np.maximum(np.maximum.accumulate(np.sqrt(NR2), axis=0),
                    np.linalg.norm(s0h.reshape(2, -1), axis=1)[None, :])
    e2 = _contraction_bound(g[t0:], beta[t0:], M2)
    ne = np.abs(np.sqrt(nrm.cpu().numpy()[:, vh].astype(np.float64)) - np.sqrt(NR2))
    assert np.all(ne <= e2 + 1e-30), f"norm error {ne.max()} (worst ratio {np.max(ne / (e2 + 1e-30)):.3f})"
    print(f"  worst snapshot error / bound {worst:.3g}, norms {np.max(ne / (e2 + 1e-30)):.3g}", flush=True)
