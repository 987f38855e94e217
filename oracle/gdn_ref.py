"""Gated DeltaNet recurrence reference: plain numpy fp64, one token at a time.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): imported by tests,
``smoke()`` and the CPU baseline of ``bench.py``, never by the product path.

The recurrence is the one [PX] prints under "Gated DeltaNet Mechanics", per
value head with state S of shape (d_k, d_v):

    S_t = alpha_t S_{t-1} + beta_t k_t (v_t - S_{t-1}^T k_t)^T
    o_t = S_t^T q_t / sqrt(d_k)

Readings where the pages are silent (each one a convention of this oracle
and of the kernel):
  * alpha_t = exp(g_t), g the log-space decay gate [PX] gives next to it;
    beta_t is the write strength (sigmoid of the b projection, [LIT]).
  * q and k enter L2-normalized per head (divided by max(|x|, 1e-6)); with
    |k| = 1 and alpha, beta in (0, 1] the map S -> alpha S - beta k k^T S has
    norm <= 1, so the state stays bounded.
  * S_0 = 0 unless a start state is given; value head h reads q/k head
    h * n_qk // n_v.
"""
from __future__ import annotations

import numpy as np

NORM_EPS = 1e-6


def l2_normalize(x: np.ndarray) -> np.ndarray:
    """x / max(|x|_2, 1e-6) along the last axis, fp64."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, NORM_EPS)


def gdn_recurrence_ref(q, k, v, g, beta, s0=None, snap_steps=()):
    """Run the recurrence over T tokens.

    q, k: [T, n_qk, d_k]; v: [T, n_v, d_v]; g, beta: [T, n_v] (g = log alpha).
    s0: [n_v, d_k, d_v] or None (zeros).  Returns (o [T, n_v, d_v], S_T, snaps
    [len(snap_steps), n_v, d_k, d_v] holding S after each listed token,
    norms [T, n_v] with |S_t|_F^2)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    T, n_qk, d_k = q.shape
    n_v, d_v = v.shape[1], v.shape[2]
    if n_v % n_qk:
        raise ValueError("value heads must be a multiple of q/k heads")
    head_of = np.arange(n_v) * n_qk // n_v
    S = np.zeros((n_v, d_k, d_v)) if s0 is None else np.array(s0, dtype=np.float64)
    o = np.empty((T, n_v, d_v))
    norms = np.empty((T, n_v))
    snaps = []
    want = set(int(s) for s in snap_steps)
    for t in range(T):
        kh = l2_normalize(k[t])[head_of]              # [n_v, d_k]
        qh = l2_normalize(q[t])[head_of]
        alpha = np.exp(g[t])                          # [n_v]
        u = np.einsum("hij,hi->hj", S, kh)            # S_{t-1}^T k
        S = alpha[:, None, None] * S + np.einsum("hi,hj->hij", kh, beta[t][:, None] * (v[t] - u))
        o[t] = np.einsum("hij,hi->hj", S, qh) / np.sqrt(d_k)
        norms[t] = np.sum(S * S, axis=(1, 2))
        if t in want:
            snaps.append(S.copy())
    return o, S, np.array(snaps).reshape(len(snaps), n_v, d_k, d_v), norms


def split_projection_rows(x, q_col, k_col, v_col, g_col, beta_col, n_qk, n_v, d=128):
    """Cut fp32 projection rows [T, ldx] into the recurrence's inputs, the
    column layout nvfp4_gdn_recurrence reads (v_col = -1: v = 0)."""
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    q = x[:, q_col:q_col + n_qk * d].reshape(T, n_qk, d)
    k = x[:, k_col:k_col + n_qk * d].reshape(T, n_qk, d)
    v = np.zeros((T, n_v, d)) if v_col < 0 else x[:, v_col:v_col + n_v * d].reshape(T, n_v, d)
    return q, k, v, x[:, g_col:g_col + n_v], x[:, beta_col:beta_col + n_v]
