"""Brute-force numpy oracle: explicit transition matrices, explicit products.

TEST INFRASTRUCTURE ONLY (see :mod:`oracle`).  Independent of the C token loop:
instead of updating a state in place, every token's d_k x d_k transition matrix
M_t is formed explicitly and the segment quantities are taken from their
definitions ([ZH] 2.1):

* T_C = M_L ... M_1, multiplied out left to right;
* S(C|0) = sum_t (M_L ... M_{t+1}) c_t k_t v_t^T, with the suffix products
  accumulated backwards from the end of the segment, so no forward state
  recurrence is involved;
* per-token outputs o_t = S_t^T (scale q_t) with S_t taken from the same
  explicit sum over the prefix [1, t].

Only for tiny inputs (d <= 32, a few hundred tokens).
"""
from __future__ import annotations

import numpy as np

GATE_HEAD, GATE_TOKEN, GATE_DIAG = 0, 1, 2


def transition(k_t, beta_t, g_t, *, gate: int, delta: int) -> np.ndarray:
    """Dense M_t = G_t (I - beta_t k_t k_t^T) (delta 1), (I - beta_t k_t k_t^T) G_t
    (delta 2: gate before the erase) or M_t = G_t (delta 0)."""
    dk = k_t.shape[0]
    E = np.eye(dk) - beta_t * np.outer(k_t, k_t) if delta else np.eye(dk)
    if gate == GATE_DIAG:
        G = np.diag(np.exp(np.asarray(g_t, dtype=np.float64)))
    else:
        G = np.exp(float(g_t)) * np.eye(dk)
    return E @ G if delta == 2 else G @ E


def _gate_of(g, t, h, gate):
    if gate == GATE_HEAD:
        return g[h]
    if gate == GATE_TOKEN:
        return g[t, h]
    return g[t, h, :]


def matrices(k, beta, g, h, t0, t1, *, gate, delta):
    k = np.asarray(k, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = None if beta is None else np.asarray(beta, dtype=np.float64)
    return [transition(k[t, h], 0.0 if beta is None else beta[t, h], _gate_of(g, t, h, gate),
                       gate=gate, delta=delta) for t in range(t0, t1)]


def segment_pair(k, v, g, beta, h, t0, t1, *, gate, delta):
    """(T_C, S(C|0)) of tokens [t0, t1) for head h, from explicit products."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dk, dv = k.shape[2], v.shape[2]
    Ms = matrices(k, beta, g, h, t0, t1, gate=gate, delta=delta)
    T = np.eye(dk)
    for M in Ms:
        T = M @ T
    S = np.zeros((dk, dv))
    suffix = np.eye(dk)  # M_L ... M_{t+1}
    for idx in range(len(Ms) - 1, -1, -1):
        t = t0 + idx
        c = float(beta[t, h]) if delta else 1.0
        S += suffix @ (c * np.outer(k[t, h], v[t, h]))
        suffix = suffix @ Ms[idx]
    return T, S


def outputs(q, k, v, g, beta, h, t0, t1, *, gate, delta, scale, S0=None):
    """Per-token outputs o_t = S_t^T (scale q_t), t in [t0, t1), for head h,
    with S_t = (M_t..M_{t0}) S0 + sum_{s<=t} (M_t..M_{s+1}) c_s k_s v_s^T
    evaluated as an explicit sum for every t (quadratic; tiny inputs only)."""
    q = np.asarray(q, dtype=np.float64)
    dv = np.asarray(v).shape[2]
    dk = np.asarray(k).shape[2]
    S0 = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, dtype=np.float64)
    out = np.empty((t1 - t0, dv))
    for t in range(t0, t1):
        T, S = segment_pair(k, v, g, beta, h, t0, t + 1, gate=gate, delta=delta)
        St = T @ S0 + S
        out[t - t0] = St.T @ (scale * q[t, h])
    return out
