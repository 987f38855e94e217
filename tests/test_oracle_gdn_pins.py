"""Pins of the Gated DeltaNet recurrence reference (oracle/gdn_ref.py), CPU
only: closed forms of single steps, the delta rule's overwrite along a key,
pure decay, the alpha = 0 limit, the norm bound that the update's
contraction gives, linearity in (S_0, v), and invariance to the scale of q
and k."""
import math

import numpy as np

from oracle import gdn_ref as G

D = 128


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_first_step_closed_form():
    rng = np.random.default_rng(1)
    q, k, v = _rand(rng, 1, 1, D), _rand(rng, 1, 1, D), _rand(rng, 1, 1, D)
    g, beta = np.array([[-0.3]]), np.array([[0.7]])
    o, S, _, norms = G.gdn_recurrence_ref(q, k, v, g, beta)
    kh = k[0, 0] / np.linalg.norm(k[0, 0])
    qh = q[0, 0] / np.linalg.norm(q[0, 0])
    assert np.allclose(S[0], 0.7 * np.outer(kh, v[0, 0]), rtol=0, atol=1e-14)
    assert np.allclose(o[0, 0], 0.7 * (kh @ qh) / math.sqrt(D) * v[0, 0], rtol=0, atol=1e-14)
    assert np.isclose(norms[0, 0], 0.49 * np.sum(v[0, 0] ** 2), rtol=1e-14)


def test_delta_rule_overwrites_along_a_key():
    # alpha = 1, beta = 1, orthonormal keys: reading along a key returns the
    # last value written along it; other keys are untouched
    e = np.eye(D)
    rng = np.random.default_rng(2)
    v1, v2, v1b = _rand(rng, D), _rand(rng, D), _rand(rng, D)
    k = np.stack([e[3], e[7], e[3]])[:, None, :] * np.array([2.0, 0.5, 3.0])[:, None, None]  # scaled keys
    v = np.stack([v1, v2, v1b])[:, None, :]
    q = np.stack([e[3], e[3], e[7]])[:, None, :]
    o, S, snaps, _ = G.gdn_recurrence_ref(q, k, v, np.zeros((3, 1)), np.ones((3, 1)), snap_steps=[1])
    assert np.allclose(snaps[0][0].T @ e[3], v1, atol=1e-13) and np.allclose(snaps[0][0].T @ e[7], v2, atol=1e-13)
    assert np.allclose(S[0].T @ e[3], v1b, atol=1e-13) and np.allclose(S[0].T @ e[7], v2, atol=1e-13)
    assert np.allclose(o[0, 0], v1 / math.sqrt(D), atol=1e-13)
    assert np.allclose(o[2, 0], v2 / math.sqrt(D), atol=1e-13)


def test_pure_decay_and_memoryless_limit():
    rng = np.random.default_rng(3)
    T = 20
    q, k, v = _rand(rng, T, 1, D), _rand(rng, T, 1, D), _rand(rng, T, 2, D)
    s0 = _rand(rng, 2, D, D)
    g = -rng.uniform(0.01, 0.2, (T, 2))
    # beta = 0: S_T = exp(sum g) S_0
    _, S, _, _ = G.gdn_recurrence_ref(q, k, v, g, np.zeros((T, 2)), s0=s0)
    assert np.allclose(S, np.exp(g.sum(0))[:, None, None] * s0, rtol=1e-12, atol=0)
    # alpha = 0 (g = -inf): the printed update keeps only the write along the
    # last key, S_T = beta_T khat_T (v_T - S_{T-1}^T khat_T)^T (rank one)
    beta = rng.uniform(0.1, 1.0, (T, 2))
    _, S, snaps, _ = G.gdn_recurrence_ref(q, k, v, np.full((T, 2), -np.inf), beta, s0=s0, snap_steps=[T - 2])
    kh = k[-1, 0] / np.linalg.norm(k[-1, 0])
    for h in range(2):
        want = beta[-1, h] * np.outer(kh, v[-1, h] - snaps[0][h].T @ kh)
        assert np.allclose(S[h], want, rtol=0, atol=1e-12)
        assert np.allclose(S[h] - np.outer(kh, kh @ S[h]), 0.0, atol=1e-12)


def test_norm_bound_from_contraction_and_head_mapping():
    rng = np.random.default_rng(4)
    T = 60
    q, k, v = _rand(rng, T, 2, D), _rand(rng, T, 2, D), _rand(rng, T, 4, D)
    g = -np.abs(rng.standard_normal((T, 4))) * 0.05
    beta = rng.uniform(0, 1, (T, 4))
    _, _, _, norms = G.gdn_recurrence_ref(q, k, v, g, beta)
    bound = np.cumsum(beta * np.linalg.norm(v, axis=2), axis=0)
    assert np.all(np.sqrt(norms) <= bound * (1 + 1e-12))
    # value heads 0 and 1 share q/k head 0, 2 and 3 share head 1: equal v and
    # gates give equal states within a pair, different across pairs
    v2 = np.repeat(v[:, :1], 4, axis=1)
    g2, b2 = np.repeat(g[:, :1], 4, axis=1), np.repeat(beta[:, :1], 4, axis=1)
    _, S, _, _ = G.gdn_recurrence_ref(q, k, v2, g2, b2)
    assert np.array_equal(S[0], S[1]) and np.array_equal(S[2], S[3]) and not np.allclose(S[0], S[2])


def test_linear_in_start_state_and_values_and_scale_free_in_q_k():
    rng = np.random.default_rng(5)
    T = 40
    q, k, v = _rand(rng, T, 1, D), _rand(rng, T, 1, D), _rand(rng, T, 1, D)
    g = -rng.uniform(0.001, 0.1, (T, 1))
    beta = rng.uniform(0, 1, (T, 1))
    s0, ds = _rand(rng, 1, D, D), _rand(rng, 1, D, D) * 0.01
    _, Sa, _, _ = G.gdn_recurrence_ref(q, k, v, g, beta, s0=s0 + ds)
    _, Sb, _, _ = G.gdn_recurrence_ref(q, k, v, g, beta, s0=s0)
    _, Sd, _, _ = G.gdn_recurrence_ref(q, k, np.zeros_like(v), g, beta, s0=ds)
    assert np.allclose(Sa - Sb, Sd, rtol=0, atol=1e-12)
    o1, S1, _, _ = G.gdn_recurrence_ref(q, k, v, g, beta)
    o2, S2, _, _ = G.gdn_recurrence_ref(q * 7.5, k * 0.02, v, g, beta)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-14) and np.allclose(S1, S2, rtol=1e-12, atol=1e-14)


def test_split_projection_rows_reads_each_part_from_its_columns():
    """Projection rows assembled from known parts (q, k, v, g, beta placed at
    chosen columns with gaps and in a scrambled order, each part holding
    values no other part holds) come back part by part; v_col = -1 gives
    v = 0.  A swapped pair of column arguments, a wrong head count or a
    transposed reshape returns another part's values and fails."""
    rng = np.random.default_rng(6)
    T, n_qk, n_v, d = 5, 2, 4, 8
    parts = {"q": rng.uniform(100, 101, (T, n_qk, d)), "k": rng.uniform(200, 201, (T, n_qk, d)),
             "v": rng.uniform(300, 301, (T, n_v, d)), "g": rng.uniform(-2, -1, (T, n_v)),
             "beta": rng.uniform(0.1, 0.9, (T, n_v))}
    # column order beta | pad | v | g | pad | k | q | pad
    order = ["beta", None, "v", "g", None, "k", "q", None]
    cols, blocks, c = {}, [], 0
    for name in order:
        blk = np.full((T, 3), -7.0) if name is None else parts[name].reshape(T, -1)
        if name is not None:
            cols[name] = c
        blocks.append(blk)
        c += blk.shape[1]
    x = np.concatenate(blocks, axis=1)
    q, k, v, g, beta = G.split_projection_rows(x, cols["q"], cols["k"], cols["v"], cols["g"], cols["beta"],
                                               n_qk, n_v, d=d)
    for name, got in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
        assert got.shape == parts[name].shape, name
        assert np.array_equal(got, parts[name]), name
    _, _, v0, g0, b0 = G.split_projection_rows(x, cols["q"], cols["k"], -1, cols["g"], cols["beta"], n_qk, n_v,
                                               d=d)
    assert v0.shape == (T, n_v, d) and not np.any(v0)
    assert np.array_equal(g0, parts["g"]) and np.array_equal(b0, parts["beta"])
