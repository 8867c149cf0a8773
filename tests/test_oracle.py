"""Pins for the fp64 CPU oracle, against facts that do not come from the oracle.

Each test checks the oracle against one of: values worked by hand from the
definition (tests/golden), the numpy brute force (explicit transition matrices,
suffix products -- no forward recurrence), closed forms (identity transition,
scalar decay, beta = 0, orthonormal keys, plain and decayed causal linear
attention), the composition law of the Chinese HYPIC page, section 2.1
(S(C1 C2) = T(C2) S(C1) + S(C2)), and invariants (contraction, naive-sum
failure).  Non-square d_k != d_v is used throughout so that a transposed
operand cannot pass.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import brute
from hybrid_attention_prefill_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_two_tokens.json")
VARIANTS = [  # (gate, delta)
    (wl.GATE_TOKEN, True),   # gated DeltaNet
    (wl.GATE_DIAG, True),    # KDA-style: diag(a)(I - b k k^T)
    (wl.GATE_HEAD, False),   # RetNet-style constant decay
    (wl.GATE_TOKEN, False),  # scalar-gated, no erase
    (wl.GATE_DIAG, False),   # per-channel gate, no erase
    (wl.GATE_HEAD, True),    # constant decay with erase
    (wl.GATE_DIAG, 2),       # KDA, gate before the erase: (I - b k k^T) diag(a)
]


def _rand(seed, N, H, dk, dv, gate, *, unit_k=True, beta_shift=0.0, g_scale=0.3):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((N, H, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((N, H, dv))
    q = rng.standard_normal((N, H, dk))
    beta = 1.0 / (1.0 + np.exp(-(rng.standard_normal((N, H)) + beta_shift)))
    if gate == wl.GATE_HEAD:
        g = -g_scale * np.abs(rng.standard_normal(H))
    elif gate == wl.GATE_TOKEN:
        g = -g_scale * np.logaddexp(0, rng.standard_normal((N, H)))
    else:
        g = -g_scale * np.logaddexp(0, rng.standard_normal((N, H, dk)))
    return q, k, v, g, beta


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ---------------------------------------------------------------- hand-worked values
def test_golden_scalar_gate_two_tokens():
    fx = json.load(open(GOLDEN))["scalar_gate"]
    k = np.array(fx["k"])[:, None, :]
    v = np.array(fx["v"])[:, None, :]
    q = np.array(fx["q"])[:, None, :]
    beta = np.array(fx["beta"])[:, None]
    g = np.log(np.array(fx["alpha"]))[:, None]
    T, S = oracle.segment_build(k, v, g, beta, [0], [2], gate=wl.GATE_TOKEN, delta=True)
    np.testing.assert_allclose(T[0, 0], fx["T"], atol=1e-14)
    np.testing.assert_allclose(S[0, 0], fx["S"], atol=1e-14)
    _, out = oracle.run(k, v, g, beta, gate=wl.GATE_TOKEN, delta=True, q=q, scale=1.0)
    np.testing.assert_allclose(out[:, 0, :], fx["outputs"], atol=1e-14)
    R = oracle.compose(T, S, [[0]], np.array(fx["prefix_state"])[None, None])
    np.testing.assert_allclose(R[0, 0], fx["composed"], atol=1e-14)


def test_golden_diagonal_gate_order():
    fx = json.load(open(GOLDEN))["diagonal_gate"]
    k = np.array(fx["k"])[:, None, :]
    v = np.array(fx["v"])[:, None, :]
    beta = np.array(fx["beta"])[:, None]
    g = np.log(np.array(fx["a"]))[:, None, :]
    T, S = oracle.segment_build(k, v, g, beta, [0], [2], gate=wl.GATE_DIAG, delta=True)
    np.testing.assert_allclose(T[0, 0], fx["T"], atol=1e-14)
    np.testing.assert_allclose(S[0, 0], fx["S"], atol=1e-14)


def test_golden_diagonal_gate_before_erase():
    fx = json.load(open(GOLDEN))["diagonal_gate_before_erase"]
    k = np.array(fx["k"])[:, None, :]
    v = np.array(fx["v"])[:, None, :]
    beta = np.array(fx["beta"])[:, None]
    g = np.log(np.array(fx["a"]))[:, None, :]
    T, S = oracle.segment_build(k, v, g, beta, [0], [2], gate=wl.GATE_DIAG, delta=2)
    np.testing.assert_allclose(T[0, 0], fx["T"], atol=1e-14)
    np.testing.assert_allclose(S[0, 0], fx["S"], atol=1e-14)
    _, S1 = oracle.segment_build(k, v, g, beta, [0], [2], gate=wl.GATE_DIAG, delta=1)
    np.testing.assert_allclose(S1[0, 0], fx["S_other_order"], atol=1e-14)


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("gate,delta", VARIANTS)
def test_build_matches_brute_force(gate, delta):
    H, dk, dv, N = 2, 8, 5, 41
    q, k, v, g, beta = _rand(11, N, H, dk, dv, gate)
    cuts = [0, 1, 17, 41]
    T, S = oracle.segment_build(k, v, g, beta, cuts[:-1], cuts[1:], gate=gate, delta=delta)
    for s in range(3):
        for h in range(H):
            Tb, Sb = brute.segment_pair(k, v, g, beta, h, cuts[s], cuts[s + 1], gate=gate, delta=delta)
            assert _rel(T[s, h], Tb) < 1e-12
            assert _rel(S[s, h], Sb) < 1e-12 or np.linalg.norm(Sb) < 1e-300


@pytest.mark.parametrize("gate,delta", VARIANTS[:3])
def test_outputs_match_brute_force(gate, delta):
    H, dk, dv, N = 2, 6, 4, 23
    q, k, v, g, beta = _rand(5, N, H, dk, dv, gate)
    S0 = np.random.default_rng(1).standard_normal((H, dk, dv))
    S, out = oracle.run(k, v, g, beta, gate=gate, delta=delta, t0=3, t1=N, S0=S0, q=q, scale=0.7)
    for h in range(H):
        ob = brute.outputs(q, k, v, g, beta, h, 3, N, gate=gate, delta=delta, scale=0.7, S0=S0[h])
        assert _rel(out[:, h, :], ob) < 1e-12
        Tb, Sb = brute.segment_pair(k, v, g, beta, h, 3, N, gate=gate, delta=delta)
        assert _rel(S[h], Tb @ S0[h] + Sb) < 1e-12


# ---------------------------------------------------------------- composition law
@pytest.mark.parametrize("gate,delta", VARIANTS)
@pytest.mark.parametrize("n_cut", [1, 2, 7])
def test_split_invariance(gate, delta, n_cut):
    """Composing the pairs of any split equals the full recurrence."""
    H, dk, dv, N = 3, 12, 7, 200
    q, k, v, g, beta = _rand(100 + n_cut, N, H, dk, dv, gate, g_scale=0.02)
    rng = np.random.default_rng(n_cut)
    cuts = np.sort(rng.choice(np.arange(1, N), size=n_cut, replace=False))
    bounds = np.concatenate([[0], cuts, [N]])
    T, S = oracle.segment_build(k, v, g, beta, bounds[:-1], bounds[1:], gate=gate, delta=delta)
    R = oracle.compose(T, S, np.arange(len(bounds) - 1)[None, :])
    S_full, _ = oracle.run(k, v, g, beta, gate=gate, delta=delta)
    for h in range(H):
        assert _rel(R[0, h], S_full[h]) < 1e-12
    # the T of the whole sequence is the ordered product of the pieces' T, later on the left
    T_all, _ = oracle.segment_build(k, v, g, beta, [0], [N], gate=gate, delta=delta)
    for h in range(H):
        P = np.eye(dk)
        for s in range(len(bounds) - 1):
            P = T[s, h] @ P
        assert _rel(T_all[0, h], P) < 1e-12


def test_compose_is_associative():
    """Left fold over a chain equals folding the chain's two halves first."""
    H, dk, dv = 2, 6, 9
    rng = np.random.default_rng(3)
    n = 9
    T = rng.standard_normal((n, H, dk, dk)) * 0.3
    S = rng.standard_normal((n, H, dk, dv))
    R0 = rng.standard_normal((1, H, dk, dv))
    left = oracle.compose(T, S, np.arange(n)[None, :], R0)
    # (T_b, S_b) o (T_a, S_a) = (T_b T_a, T_b S_a + S_b), folded over each half
    def fold(ids):
        Ta = np.broadcast_to(np.eye(dk), (H, dk, dk)).copy()
        Sa = np.zeros((H, dk, dv))
        for i in ids:
            Ta = T[i] @ Ta
            Sa = T[i] @ Sa + S[i]
        return Ta, Sa
    T1, S1 = fold(range(4))
    T2, S2 = fold(range(4, n))
    Tc, Sc = T2 @ T1, T2 @ S1 + S2
    assert _rel(left[0], Tc @ R0[0] + Sc) < 1e-12


def test_skipped_steps_and_scalar_T_layout():
    H, dk, dv = 2, 4, 3
    rng = np.random.default_rng(9)
    t = rng.uniform(0.2, 0.9, size=(5, H))
    S = rng.standard_normal((5, H, dk, dv))
    ids = np.array([[0, -1, 3, 4, -1]])
    dense = t[:, :, None, None] * np.eye(dk)
    a = oracle.compose(t, S, ids, t_scalar=True)
    b = oracle.compose(dense, S, ids)
    ref = np.zeros((H, dk, dv))
    for i in (0, 3, 4):
        ref = t[i][:, None, None] * ref + S[i]
    assert _rel(a[0], ref) < 1e-14 and _rel(b[0], ref) < 1e-14


def test_compose_gemm_matches_token_loop():
    """The matrix-product composition equals the C routine's on chains with skipped and
    repeated pairs, several heads, d_k != d_v and a nonzero starting state."""
    H, dk, dv, n_pair = 3, 7, 5, 6
    rng = np.random.default_rng(31)
    T = rng.standard_normal((n_pair, H, dk, dk)) * 0.4
    S = rng.standard_normal((n_pair, H, dk, dv))
    ids = rng.integers(-1, n_pair, size=(4, 23))
    R0 = rng.standard_normal((4, H, dk, dv))
    a = oracle.compose(T, S, ids, R0)
    b = oracle.compose_gemm(T, S, ids, R0, workers=3)
    assert _rel(b, a).max() < 1e-13
    assert np.array_equal(oracle.compose_gemm(T, S, np.full((2, 4), -1), R0[:2]), R0[:2])


@pytest.mark.parametrize("gate,delta", [(wl.GATE_TOKEN, True), (wl.GATE_DIAG, True)])
def test_compose_gemm_split_invariance(gate, delta):
    """Pairs of a cut sequence composed by the matrix-product routine give the full
    recurrence's state (the composition law, [ZH] 2.1), and the identity transition gives
    the plain sum of the states."""
    H, dk, dv, N = 2, 6, 4, 70
    _, k, v, g, beta = _rand(33, N, H, dk, dv, gate)
    bounds = [0, 9, 30, 31, 70]
    T, S = oracle.segment_build(k, v, g, beta, bounds[:-1], bounds[1:], gate=gate, delta=delta)
    full, _ = oracle.run(k, v, g, beta, gate=gate, delta=delta)
    R = oracle.compose_gemm(T, S, [list(range(4))])
    assert _rel(R[0], full).max() < 1e-12
    I = np.broadcast_to(np.eye(dk), T.shape).copy()
    assert _rel(oracle.compose_gemm(I, S, [[0, 2, 3]])[0], S[0] + S[2] + S[3]).max() < 1e-14


# ---------------------------------------------------------------- closed forms
def test_identity_transition_gives_plain_sum():
    """Plain linear attention (no gate, no erase): T = I exactly, S = K^T V, and the
    naive sum of zero-initial states is exact ([ZH] 2.1 says so for this case)."""
    H, dk, dv, N = 2, 8, 5, 60
    q, k, v, _, _ = _rand(21, N, H, dk, dv, wl.GATE_HEAD)
    g = np.zeros(H)
    bounds = [0, 25, 60]
    T, S = oracle.segment_build(k, v, g, None, bounds[:-1], bounds[1:], gate=wl.GATE_HEAD, delta=False)
    assert np.array_equal(T, np.broadcast_to(np.eye(dk), T.shape))
    for s in range(2):
        ref = np.einsum("th,tn->hn", k[bounds[s]:bounds[s + 1], 0], v[bounds[s]:bounds[s + 1], 0])
        assert _rel(S[s, 0], ref) < 1e-13
    R = oracle.compose(T, S, [[0, 1]])
    assert _rel(R, oracle.naive_sum(S, [[0, 1]])) < 1e-14


@pytest.mark.parametrize("h", range(8))
def test_retnet_closed_form(h):
    """Constant decay gamma: T_C = gamma^L I and S(C|0) = sum_t gamma^(L-1-t) k_t v_t^T."""
    W = wl.make("retnet-8h-d64", n_heads=8, n_seg=2, seg_len=96)
    T, S = oracle.segment_build(W.k, W.v, W.g, None, W.cache_begin, W.cache_end,
                                gate=W.gate, delta=W.delta)
    gam = math.exp(float(W.g[h]))
    for s in range(2):
        b, e = W.cache_begin[s], W.cache_end[s]
        L = e - b
        assert _rel(T[s, h], gam ** L * np.eye(W.d_k)) < 1e-13
        w_ = gam ** (L - 1 - np.arange(L))
        ref = (W.k[b:e, h].astype(np.float64) * w_[:, None]).T @ W.v[b:e, h].astype(np.float64)
        assert _rel(S[s, h], ref) < 1e-12


def test_beta_zero_reduces_to_scalar_decay():
    H, dk, dv, N = 2, 8, 6, 50
    q, k, v, g, _ = _rand(31, N, H, dk, dv, wl.GATE_TOKEN)
    beta = np.zeros((N, H))
    T, S = oracle.segment_build(k, v, g, beta, [0], [N], gate=wl.GATE_TOKEN, delta=True)
    for h in range(H):
        assert _rel(T[0, h], math.exp(g[:, h].sum()) * np.eye(dk)) < 1e-13
        assert np.all(S[0, h] == 0)


def test_orthonormal_keys_closed_form():
    """With orthonormal keys the erase factors commute:
    T = exp(sum g) (I - sum_t beta_t k_t k_t^T), S = sum_t exp(sum_{s>t} g_s) beta_t k_t v_t^T."""
    dk, dv, L = 16, 5, 10
    rng = np.random.default_rng(41)
    Q, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Q[:, :L].T[:, None, :]
    v = rng.standard_normal((L, 1, dv))
    beta = rng.uniform(0.05, 0.95, size=(L, 1))
    g = -rng.uniform(0.0, 0.5, size=(L, 1))
    T, S = oracle.segment_build(k, v, g, beta, [0], [L], gate=wl.GATE_TOKEN, delta=True)
    Tref = math.exp(g.sum()) * (np.eye(dk) - sum(beta[t, 0] * np.outer(k[t, 0], k[t, 0]) for t in range(L)))
    Sref = sum(math.exp(g[t + 1:, 0].sum()) * beta[t, 0] * np.outer(k[t, 0], v[t, 0]) for t in range(L))
    assert _rel(T[0, 0], Tref) < 1e-13
    assert _rel(S[0, 0], Sref) < 1e-13


def test_plain_causal_linear_attention_outputs():
    """No gate, no erase: o_t = scale * sum_{s<=t} (k_s . q_t) v_s = scale * tril(Q K^T) V."""
    H, dk, dv, N = 1, 7, 4, 30
    q, k, v, _, _ = _rand(51, N, H, dk, dv, wl.GATE_HEAD)
    _, out = oracle.run(k, v, np.zeros(H), None, gate=wl.GATE_HEAD, delta=False, q=q, scale=0.5)
    ref = 0.5 * np.tril(q[:, 0] @ k[:, 0].T) @ v[:, 0]
    assert _rel(out[:, 0], ref) < 1e-13


def test_retention_parallel_form_outputs():
    """Constant decay: o_t = scale * sum_{s<=t} gamma^(t-s) (k_s . q_t) v_s (retention's parallel form)."""
    H, dk, dv, N = 1, 7, 4, 30
    q, k, v, _, _ = _rand(52, N, H, dk, dv, wl.GATE_HEAD)
    gam = 0.93
    _, out = oracle.run(k, v, np.array([math.log(gam)]), None, gate=wl.GATE_HEAD, delta=False, q=q, scale=0.5)
    t = np.arange(N)
    D = np.where(t[:, None] >= t[None, :], gam ** (t[:, None] - t[None, :]), 0.0)
    ref = 0.5 * ((q[:, 0] @ k[:, 0].T) * D) @ v[:, 0]
    assert _rel(out[:, 0], ref) < 1e-13


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("gate", [wl.GATE_TOKEN, wl.GATE_DIAG])
def test_transition_product_is_a_contraction(gate):
    H, dk, dv, N = 4, 16, 4, 300
    q, k, v, g, beta = _rand(61, N, H, dk, dv, gate, g_scale=0.01)
    T, _ = oracle.segment_build(k, v, g, beta, [0, 100], [100, 300], gate=gate, delta=True)
    assert np.max(np.linalg.norm(T, ord=2, axis=(-2, -1))) <= 1.0 + 1e-12


def test_naive_sum_closed_form_and_failure():
    """Two RetNet segments: the naive sum drops T(C2), so its error is
    ||(1 - gamma^L2) S1|| / ||gamma^L2 S1 + S2||, at least five times the bf16 tolerance on every head."""
    W = wl.make("retnet-8h-d64", n_heads=8, n_seg=2, seg_len=256)
    T, S = oracle.segment_build(W.k, W.v, W.g, None, W.cache_begin, W.cache_end,
                                gate=W.gate, delta=W.delta)
    good = oracle.compose(T, S, [[0, 1]])[0]
    naive = oracle.naive_sum(S, [[0, 1]])[0]
    for h in range(8):
        gL = math.exp(float(W.g[h])) ** 256
        closed = np.linalg.norm((1 - gL) * S[0, h]) / np.linalg.norm(gL * S[0, h] + S[1, h])
        err = np.linalg.norm(naive[h] - good[h]) / np.linalg.norm(good[h])
        assert abs(err - closed) < 1e-10 * max(closed, 1.0)
        assert err > 5 * 5e-3   # several times the bf16 parity tolerance


def test_naive_sum_loses_the_decayed_prefix():
    """If C2 writes nothing, the naive sum's error relative to the prefix state is
    1 - gamma^L2: 0.2213 for gamma = 1 - 2^-10 over 256 tokens, one reading of
    the 22% slow-head figure the pages quote."""
    W = wl.make("retnet-8h-d64", n_heads=8, n_seg=2, seg_len=256)
    v = W.v.copy()
    v[256:] = 0.0
    T, S = oracle.segment_build(W.k, v, W.g, None, W.cache_begin, W.cache_end,
                                gate=W.gate, delta=W.delta)
    good = oracle.compose(T, S, [[0, 1]])[0]
    naive = oracle.naive_sum(S, [[0, 1]])[0]
    h = 5  # gamma = 1 - 2^-10
    err = np.linalg.norm(naive[h] - good[h]) / np.linalg.norm(S[0, h])
    assert abs(err - (1 - (1 - 2.0 ** -10) ** 256)) < 1e-6
    assert abs(err - 0.2213) < 5e-4


# ---------------------------------------------------------------- seam windows
@pytest.mark.parametrize("gate", [wl.GATE_TOKEN, wl.GATE_DIAG])
def test_seam_chain_equals_full_recurrence(gate):
    """Seam windows stepped from the running state, then the cached pair of the rest of
    each segment: the final state and the window outputs equal the full recurrence's."""
    H, dk, dv, w = 2, 8, 6, 4
    lens = [30, 25, 41, 17]
    N = sum(lens)
    q, k, v, g, beta = _rand(71, N, H, dk, dv, gate, g_scale=0.05)
    starts = np.concatenate([[0], np.cumsum(lens)])
    cb = starts[:-1].copy()
    cb[1:] += w
    T, S = oracle.segment_build(k, v, g, beta, cb, starts[1:], gate=gate, delta=True)
    seam = starts[:-1].copy()[None, :]
    seam[0, 0] = -1
    R, out = oracle.seam_advance(q, k, v, g, beta, seam, gate=gate, delta=True, w=w, scale=0.3,
                                 pair_id=np.arange(4)[None, :], T_cache=T, S_cache=S)
    S_full, o_full = oracle.run(k, v, g, beta, gate=gate, delta=True, q=q, scale=0.3)
    assert _rel(R[0], S_full) < 1e-12
    assert np.all(np.isnan(out[0, 0]))
    for j in range(1, 4):
        ref = o_full[starts[j]:starts[j] + w]
        assert _rel(out[0, j], ref) < 1e-12
