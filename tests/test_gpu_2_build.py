"""hypic_segment_build parity with the fp64 oracle.

Tolerances: relative Frobenius error per (segment, head) <= 1e-4 for fp32
inputs and <= 5e-3 for bf16 inputs (fp32 state; the oracle is fed the same
bf16-rounded values).  T below 1e-30 in norm is held to the floor rule.
"""
import numpy as np
import pytest
import torch

import oracle
from hybrid_attention_prefill_amd import binding as hb
from hybrid_attention_prefill_amd import workloads as wl
from _util import assert_pairs_close, dev, rel_f, t_split, t_value, workload_tensors

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 5e-3}


def _gpu_build(W, t_layout=hb.T_DENSE, begin=None, end=None):
    x = workload_tensors(W)
    b = W.cache_begin if begin is None else begin
    e = W.cache_end if end is None else end
    T, S = hb.segment_build(x["k"], x["v"], x["g"], x["beta"], dev(b, torch.int64), dev(e, torch.int64),
                            gate=W.gate, delta=W.delta, t_layout=t_layout)
    torch.cuda.synchronize()
    return T.cpu().numpy(), S.cpu().numpy()


def _oracle_build(W, begin=None, end=None):
    b = W.cache_begin if begin is None else begin
    e = W.cache_end if end is None else end
    return oracle.segment_build(W.k, W.v, W.g, W.beta, b, e, gate=W.gate, delta=W.delta)


@pytest.mark.parametrize("stress", [False, True])
def test_tiny_gdn_fp32(stress):
    """1 head, d=16, 2 x 64 tokens, fp32: pairs, composition and the full recurrence."""
    W = wl.make("gdn-tiny-f32", stress=stress)
    print(W.name, flush=True)
    T, S = _gpu_build(W)
    T0, S0 = _oracle_build(W)
    assert_pairs_close(T, S, T0, S0, TOL["f32"], W.name)
    Rg = torch.zeros((1, 1, 16, 16), device="cuda")
    hb.compose(dev(T, torch.float32), dev(S, torch.float32), dev(W.pair_id, torch.int32), Rg)
    torch.cuda.synchronize()
    full, _ = oracle.run(W.k, W.v, W.g, W.beta, gate=W.gate, delta=W.delta)
    assert rel_f(Rg.cpu().numpy()[0], full).max() <= TOL["f32"]


@pytest.mark.parametrize("t_layout", [hb.T_SCALAR, hb.T_DENSE])
def test_retnet_full(t_layout):
    """RetNet-style decay, 8 heads, d=64, 16 x 512 (full size): T = gamma^L I,
    S by the oracle, and the ordered composition against the full recurrence."""
    W = wl.make("retnet-8h-d64")
    print(W.name, t_layout, flush=True)
    T, S = _gpu_build(W, t_layout=t_layout)
    T0, S0 = _oracle_build(W)
    if t_layout == hb.T_SCALAR:
        gam = np.exp(W.g.astype(np.float64))
        L = (W.cache_end - W.cache_begin)[:, None]
        assert np.max(np.abs(T / gam[None, :] ** L - 1)) < 1e-5
    else:
        assert_pairs_close(T, S, T0, S0, TOL["bf16"], W.name)
    assert rel_f(S, S0).max() <= TOL["bf16"]
    Rg = torch.zeros((1, 8, 64, 64), device="cuda")
    hb.compose(dev(T, torch.float32), dev(S, torch.float32), dev(W.pair_id, torch.int32), Rg, t_layout=t_layout)
    torch.cuda.synchronize()
    full, _ = oracle.run(W.k, W.v, W.g, None, gate=W.gate, delta=False)
    assert rel_f(Rg.cpu().numpy()[0], full).max() <= TOL["bf16"]


@pytest.mark.parametrize("stress", [False, True])
def test_gdn_d128_ragged(stress):
    """GDN d=128, bf16: segments spanning several chunks with ragged tails,
    a one-token segment and an empty one."""
    lens = [1024, 700, 129, 1, 65]
    W = wl.make("gdn-16h-d128-32k", stress=stress, n_heads=3, lengths=lens)
    begin = np.concatenate([W.cache_begin, [5]])
    end = np.concatenate([W.cache_end, [5]])          # empty range -> identity pair
    print(W.name, "ragged", flush=True)
    T, S = _gpu_build(W, begin=begin, end=end)
    T0, S0 = _oracle_build(W, begin=begin, end=end)
    assert_pairs_close(T, S, T0, S0, TOL["bf16"], W.name)
    assert np.array_equal(T[-1], np.broadcast_to(np.eye(128, dtype=np.float32), T[-1].shape))
    assert np.all(S[-1] == 0)


def test_gdn_stress_compose_needs_T():
    """Stress variant: composing the GPU pairs matches the full recurrence while the
    naive sum does not, so T is genuinely tested."""
    W = wl.make("gdn-16h-d128-32k", stress=True, n_heads=2, n_seg=4, seg_len=512)
    T, S = _gpu_build(W)
    Rg = torch.zeros((1, 2, 128, 128), device="cuda")
    hb.compose(dev(T, torch.float32), dev(S, torch.float32), dev(W.pair_id, torch.int32), Rg)
    torch.cuda.synchronize()
    full, _ = oracle.run(W.k, W.v, W.g, W.beta, gate=W.gate, delta=True)
    assert rel_f(Rg.cpu().numpy()[0], full).max() <= TOL["bf16"]
    naive = oracle.naive_sum(S, W.pair_id)[0]
    assert rel_f(naive, full).min() > 20 * TOL["bf16"]


def test_prefix_independence_bit_identical():
    """A segment's pair does not depend on where it sits in the packed batch or on
    its neighbours: bit-identical results for the same tokens at another offset."""
    W = wl.make("gdn-16h-d128-32k", n_heads=2, n_seg=3, seg_len=300)
    x = workload_tensors(W)
    n = W.n_tokens
    # second copy: the same tokens shifted behind a 77-token prefix of other tokens
    perm = np.random.default_rng(0).permutation(n)[:77]
    k2 = torch.cat([x["k"][perm], x["k"]])
    v2 = torch.cat([x["v"][perm], x["v"]])
    g2 = torch.cat([x["g"][perm], x["g"]])
    b2 = torch.cat([x["beta"][perm], x["beta"]])
    T1, S1 = hb.segment_build(x["k"], x["v"], x["g"], x["beta"], dev(W.cache_begin, torch.int64),
                              dev(W.cache_end, torch.int64), gate=W.gate, delta=True)
    T2, S2 = hb.segment_build(k2, v2, g2, b2, dev(W.cache_begin[::-1] + 77, torch.int64),
                              dev(W.cache_end[::-1] + 77, torch.int64), gate=W.gate, delta=True)
    torch.cuda.synchronize()
    assert torch.equal(T1, T2.flip(0)) and torch.equal(S1, S2.flip(0))


@pytest.mark.slow
def test_gdn_32k_full_size_sampled():
    """Full GDN workload (16 heads, 32 x 1024, d=128) in the benchmark's launch
    configuration; sampled (segment, head) pairs checked against the oracle."""
    W = wl.make("gdn-16h-d128-32k")
    print(W.name, "full", flush=True)
    T, S = _gpu_build(W)
    assert np.all(np.isfinite(S)) and np.all(np.isfinite(T))
    rng = np.random.default_rng(1)
    for s, h in zip(rng.integers(0, 32, 6), rng.integers(0, 16, 6)):
        b, e = W.cache_begin[s], W.cache_end[s]
        T0, S0 = oracle.segment_build(W.k[b:e, h:h + 1], W.v[b:e, h:h + 1], W.g[b:e, h:h + 1],
                                      W.beta[b:e, h:h + 1], [0], [e - b], gate=W.gate, delta=True)
        assert_pairs_close(T[s:s + 1, h:h + 1], S[s:s + 1, h:h + 1], T0, S0, TOL["bf16"], f"seg {s} head {h}")


@pytest.mark.parametrize("stress", [False, True])
def test_kda_ragged(stress):
    """KDA-style per-channel gate, d=128, bf16: several chunks, ragged tails, one token."""
    W = wl.make("kda-32h-d128-131k", stress=stress, n_heads=2, lengths=[256, 100, 33, 1], n_req=1, n_step=1, n_layers=1)
    print(W.name, "ragged", flush=True)
    T, S = _gpu_build(W)
    T0, S0 = _oracle_build(W)
    eS, eT = assert_pairs_close(T, S, T0, S0, TOL["bf16"], W.name)
    print(f"{W.name}: S {eS:.2e} T {eT}")


@pytest.mark.parametrize("gate_first", [False, True])
def test_kda_ragged_tails_after_T_is_dropped(gate_first):
    """KDA segments long enough for T to be dropped (after a few chunks on the default gates)
    that end in a partial chunk, so the chunks after the drop -- staged during the previous
    chunk by the waves that held T -- include ragged tails: 300, 1000 and 2050 tokens, and a
    segment of exactly 7 chunks.  Every (segment, head) against the oracle."""
    W = wl.make("kda-32h-d128-131k", gate_first=gate_first, n_heads=2, lengths=[300, 1000, 2050, 224],
                n_req=1, n_step=1, n_layers=1)
    print(W.name, "ragged tails after the drop", flush=True)
    T, S = _gpu_build(W)
    T0, S0 = _oracle_build(W)
    eS, _ = assert_pairs_close(T, S, T0, S0, TOL["bf16"], W.name)
    print(f"S rel_F max {eS:.2e}")


@pytest.mark.parametrize("switch", [1024, 1040])
def test_kda_decay_weakens_after_T_is_dropped(switch):
    """KDA segments of 2048 tokens whose gates decay strongly up to token `switch` (T falls
    below the floor and is dropped within the first chunks) and weakly after it (chunk decay
    factors near 1).  The chunks after the switch take the S-only path without the
    strong-decay operand precision (single bf16 Gram operands, single fp16 inverses), which
    holds only while every chunk decay factor is below 2^-8; S is checked against the oracle
    for every (segment, head)."""
    W = wl.make("kda-32h-d128-131k", n_heads=2, n_seg=2, n_req=1, n_step=1, n_layers=1)
    g = np.array(W.g, dtype=np.float64)
    for b, e in zip(W.cache_begin, W.cache_end):
        g[b + switch:e] *= 1e-3
    W.g = wl._finish(g, "bf16")
    print(W.name, "weak after", switch, flush=True)
    T, S = _gpu_build(W)
    T0, S0 = _oracle_build(W)
    assert np.all(np.sqrt(np.sum(T0.astype(np.float64) ** 2, axis=(-2, -1))) < 1e-30)   # T dropped
    eS, _ = assert_pairs_close(T, S, T0, S0, TOL["bf16"], f"{W.name} weak after {switch}")
    print(f"S rel_F max {eS:.2e}")


def test_kda_stress_compose_matches_full():
    W = wl.make("kda-32h-d128-131k", stress=True, n_heads=2, n_seg=4, seg_len=300, n_req=1, n_step=1, n_layers=1)
    T, S = _gpu_build(W)
    Rg = torch.zeros((1, 2, 128, 128), device="cuda")
    hb.compose(dev(T, torch.float32), dev(S, torch.float32), dev(np.arange(4, dtype=np.int32)[None, :], torch.int32), Rg)
    torch.cuda.synchronize()
    full, _ = oracle.run(W.k, W.v, W.g, W.beta, gate=W.gate, delta=True)
    assert rel_f(Rg.cpu().numpy()[0], full).max() <= TOL["bf16"]
    naive = oracle.naive_sum(S, np.arange(4)[None, :])[0]
    assert rel_f(naive, full).min() > 20 * TOL["bf16"]


def test_kda_segment_shape_all_heads_sampled():
    """32 heads x 2048-token segments (the KDA workload's segment shape), sampled checks."""
    W = wl.make("kda-32h-d128-131k", n_seg=3, n_req=1, n_step=1, n_layers=1)
    print(W.name, "32 heads x 3 x 2048", flush=True)
    T, S = _gpu_build(W)
    assert np.all(np.isfinite(S)) and np.all(np.isfinite(T))
    for s, h in [(0, 0), (1, 17), (2, 31)]:
        b, e = W.cache_begin[s], W.cache_end[s]
        T0, S0 = oracle.segment_build(W.k[b:e, h:h + 1], W.v[b:e, h:h + 1], W.g[b:e, h:h + 1],
                                      W.beta[b:e, h:h + 1], [0], [e - b], gate=W.gate, delta=True)
        assert_pairs_close(T[s:s + 1, h:h + 1], S[s:s + 1, h:h + 1], T0, S0, TOL["bf16"], f"seg {s} head {h}")


@pytest.mark.parametrize("name,kw", [
    ("gdn-tiny-f32", dict(stress=True)),
    ("retnet-8h-d64", dict(n_seg=3, seg_len=200)),
    ("gdn-16h-d128-32k", dict(n_heads=2, lengths=[300, 65, 1])),
    ("kda-32h-d128-131k", dict(n_heads=2, lengths=[100, 33], n_req=1, n_step=1, n_layers=1)),
])
def test_split_T_layout(name, kw):
    """T emitted as bf16 hi/lo planes (the layout the composition kernels read): the
    planes are exactly the round-to-nearest-even split of the fp32 T the same kernel
    writes in the dense layout, S is bit-identical, and hi + lo matches the oracle."""
    W = wl.make(name, **kw)
    print(W.name, "split T", flush=True)
    x = workload_tensors(W)
    sb, se = dev(W.cache_begin, torch.int64), dev(W.cache_end, torch.int64)
    T32, S32 = hb.segment_build(x["k"], x["v"], x["g"], x["beta"], sb, se, gate=W.gate, delta=W.delta)
    Tsp, Ssp = hb.segment_build(x["k"], x["v"], x["g"], x["beta"], sb, se, gate=W.gate, delta=W.delta,
                                t_layout=hb.T_SPLIT)
    torch.cuda.synchronize()
    assert Tsp.dtype == torch.bfloat16 and tuple(Tsp.shape) == (W.n_seg, W.n_heads, 2, W.d_k * W.d_k)
    assert torch.equal(Ssp, S32)
    ref = t_split(T32)
    normal = (t_split(T32.abs() >= 1e-30).float() > 0)            # fp32 normal range: exact split
    normal[..., 1, :] = normal[..., 0, :]
    assert torch.equal(Tsp[normal], ref[normal])
    t64 = T32.double().cpu().numpy()
    assert np.all(np.abs(t_value(Tsp) - t64) <= 2.0 ** -16 * np.abs(t64) + 1e-37)   # hi + lo carries 16 bits
    T0, S0 = _oracle_build(W)
    tol = TOL["f32"] if W.in_dtype == "f32" else TOL["bf16"]
    assert_pairs_close(t_value(Tsp), Ssp.cpu().numpy(), T0, S0, tol, W.name)


def _build_ws(W, begin, end, workspace, t_layout=hb.T_DENSE, want_T=True):
    x = workload_tensors(W)
    T, S = hb.segment_build(x["k"], x["v"], x["g"], x["beta"], dev(begin, torch.int64), dev(end, torch.int64),
                            gate=W.gate, delta=W.delta, t_layout=t_layout, want_T=want_T, workspace=workspace)
    torch.cuda.synchronize()
    return T, S


@pytest.mark.parametrize("d", [64, 128])
def test_cut_segments_match_oracle(d):
    """Segments longer than 16 chunks are cut into pieces built in parallel and folded by
    composition: lengths on both sides of the cut points (1024 = 16 chunks, 1025, 1771 = 28
    chunks with a ragged tail, 2100 = 3 pieces), short and empty segments in the same call."""
    lens = [1771, 2100, 1024, 1025, 64, 1, 1100]
    W = wl.make("gdn-16h-d128-32k", stress=True, n_heads=3, d=d, lengths=lens)
    begin = np.concatenate([W.cache_begin, [9]])
    end = np.concatenate([W.cache_end, [9]])
    assert hb.build_workspace_bytes(3, d, d, len(begin), W.n_tokens) > 0
    print(W.name, d, "cut", flush=True)
    T, S = _build_ws(W, begin, end, "auto")
    T0, S0 = oracle.segment_build(W.k, W.v, W.g, W.beta, begin, end, gate=W.gate, delta=W.delta)
    assert_pairs_close(T.cpu().numpy(), S.cpu().numpy(), T0, S0, TOL["bf16"], W.name)
    assert np.array_equal(T[-1].cpu().numpy(), np.broadcast_to(np.eye(d, dtype=np.float32), T[-1].shape))
    # uncut segments are bit-identical with and without the workspace
    Tu, Su = _build_ws(W, begin, end, None)
    short = [2, 4, 5, 7]
    assert torch.equal(T[short], Tu[short]) and torch.equal(S[short], Su[short])
    assert not torch.equal(S[0], Su[0])     # the cut segment took the other path


def test_cut_segments_split_T_and_S_only():
    """Cut segments with T cached as bf16 hi/lo planes, and with T not requested."""
    W = wl.make("gdn-16h-d128-32k", stress=True, n_heads=2, lengths=[1771, 300, 2000])
    print(W.name, "cut split-T", flush=True)
    T0, S0 = oracle.segment_build(W.k, W.v, W.g, W.beta, W.cache_begin, W.cache_end, gate=W.gate, delta=W.delta)
    Tsp, Ssp = _build_ws(W, W.cache_begin, W.cache_end, "auto", t_layout=hb.T_SPLIT)
    assert_pairs_close(t_value(Tsp), Ssp.cpu().numpy(), T0, S0, TOL["bf16"], W.name)
    Tn, Sn = _build_ws(W, W.cache_begin, W.cache_end, "auto", want_T=False)
    assert Tn is None and torch.equal(Sn, Ssp)


def test_cut_segment_independent_of_neighbours():
    """A cut segment's pair is bit-identical whatever the other segments of the call and
    its offset in the packed arrays."""
    W = wl.make("gdn-16h-d128-32k", n_heads=2, lengths=[1900, 700, 1000])
    x = workload_tensors(W)
    sb, se = W.cache_begin, W.cache_end
    T1, S1 = hb.segment_build(x["k"], x["v"], x["g"], x["beta"], dev(sb, torch.int64), dev(se, torch.int64),
                              gate=W.gate, delta=True)
    pre = 333
    cat = lambda a: torch.cat([a[-pre:], a])
    T2, S2 = hb.segment_build(cat(x["k"]), cat(x["v"]), cat(x["g"]), cat(x["beta"]),
                              dev(sb[:1] + pre, torch.int64), dev(se[:1] + pre, torch.int64), gate=W.gate, delta=True)
    torch.cuda.synchronize()
    assert torch.equal(T1[:1], T2) and torch.equal(S1[:1], S2)


def test_overlapping_segments_beyond_workspace_built_uncut():
    """Overlapping ranges can ask for more pieces than the workspace holds (it is sized for
    disjoint segments): the segments that do not fit are built uncut, every pair is still right."""
    W = wl.make("gdn-16h-d128-32k", stress=True, n_heads=2, lengths=[1800])
    begin = np.array([0, 0, 5, 0], dtype=np.int64)
    end = np.array([1800, 1800, 1795, 1800], dtype=np.int64)
    print(W.name, "overlap", flush=True)
    T, S = _build_ws(W, begin, end, "auto")
    T0, S0 = oracle.segment_build(W.k, W.v, W.g, W.beta, begin, end, gate=W.gate, delta=W.delta)
    assert_pairs_close(T.cpu().numpy(), S.cpu().numpy(), T0, S0, TOL["bf16"], W.name)
    Tu, Su = _build_ws(W, begin, end, None)
    assert not torch.equal(S[0], Su[0]) and torch.equal(S[3], Su[3])   # first cut, last uncut


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("stress", [False, True])
@pytest.mark.parametrize("want_T", [True, False])
def test_prefill_outputs(d, stress, want_T):
    """Cold prefill of each segment in isolation: every token's output S_t^T (scale q_t)
    and the pair, against the oracle's recurrence per segment (several chunks, ragged
    tails, one token, an empty segment); tokens outside the segments stay untouched."""
    lens = [300, 129, 1, 64, 200]
    W = wl.make("gdn-16h-d128-32k", stress=stress, n_heads=3, d=d, lengths=lens)
    # segments [0, 300) [307, 436) [436, 437) [437, 501) [501, 694) and an empty one;
    # tokens [300, 307) belong to none
    begin = np.array([0, 307, 436, 437, 501, 436], dtype=np.int64)
    end = np.array([300, 436, 437, 501, 694, 436], dtype=np.int64)
    assert W.n_tokens == 694
    x = workload_tensors(W)
    out0 = torch.full((W.n_tokens, 3, d), 7.0, device="cuda")
    print(W.name, d, "prefill", stress, want_T, flush=True)
    T, S, out = hb.segment_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], dev(begin, torch.int64),
                                   dev(end, torch.int64), scale=W.scale, want_T=want_T, out=out0)
    torch.cuda.synchronize()
    T0, S0 = oracle.segment_build(W.k, W.v, W.g, W.beta, begin, end, gate=W.gate, delta=W.delta)
    assert_pairs_close(T.cpu().numpy() if want_T else None, S.cpu().numpy(), T0, S0, TOL["bf16"], W.name)
    o = out.cpu().numpy().astype(np.float64)
    for b, e in zip(begin, end):
        if e == b:
            continue
        _, ref = oracle.run(W.k, W.v, W.g, W.beta, gate=W.gate, delta=W.delta, t0=b, t1=e, q=W.q, scale=W.scale)
        # per head and per block of 16 tokens (a single wrong token moves its block's error)
        for t0 in range(0, e - b, 16):
            blk = slice(t0, min(t0 + 16, e - b))
            err = np.linalg.norm(o[b:e][blk] - ref[blk], axis=(0, 2)) / np.linalg.norm(ref[blk], axis=(0, 2))
            assert err.max() <= TOL["bf16"], f"segment [{b}, {e}) tokens {t0}..: output rel_F {err.max():.2e}"
    assert np.all(o[300:307] == 7.0)


@pytest.mark.parametrize("dk,dv,want_T", [(64, 128, True), (64, 128, False), (128, 64, True)])
def test_prefill_rectangular_state(dk, dv, want_T):
    """Cold prefill with d_k != d_v: 64 x 128 in two column blocks of 64 value columns,
    128 x 64 in one launch with the missing value columns read as zeros; every token's
    output per 16-token block and the pairs against the oracle's recurrence per segment;
    tokens outside the segments untouched."""
    rng = np.random.default_rng(4242 + want_T + dk)
    H = 2
    begin = np.array([0, 307, 436, 437, 436], dtype=np.int64)
    end = np.array([300, 436, 437, 600, 436], dtype=np.int64)
    N = 600
    unit = lambda a: a / np.linalg.norm(a, axis=-1, keepdims=True)
    q = wl.round_bf16(rng.standard_normal((N, H, dk)))
    k = wl.round_bf16(unit(rng.standard_normal((N, H, dk))))
    v = wl.round_bf16(rng.standard_normal((N, H, dv)))
    g = wl.round_bf16(-0.1 * np.logaddexp(0.0, rng.standard_normal((N, H))))
    beta = wl.round_bf16(1.0 / (1.0 + np.exp(-rng.standard_normal((N, H)))))
    bf = torch.bfloat16
    out0 = torch.full((N, H, dv), 7.0, device="cuda")
    print("prefill rectangular", dk, dv, want_T, flush=True)
    scale = 1.0 / np.sqrt(dk)
    T, S, out = hb.segment_prefill(dev(q, bf), dev(k, bf), dev(v, bf), dev(g, bf), dev(beta, bf),
                                   dev(begin, torch.int64), dev(end, torch.int64), scale=scale,
                                   want_T=want_T, out=out0)
    torch.cuda.synchronize()
    T0, S0 = oracle.segment_build(k, v, g, beta, begin, end, gate=hb.GATE_TOKEN, delta=1)
    assert_pairs_close(t_value(T, dk) if want_T else None, S.cpu().numpy(), T0, S0, TOL["bf16"], f"{dk}x{dv}")
    o = out.cpu().numpy().astype(np.float64)
    for b, e in zip(begin, end):
        if e == b:
            continue
        _, ref = oracle.run(k, v, g, beta, gate=hb.GATE_TOKEN, delta=1, t0=b, t1=e, q=q, scale=scale)
        for t0 in range(0, e - b, 16):
            blk = slice(t0, min(t0 + 16, e - b))
            err = np.linalg.norm(o[b:e][blk] - ref[blk], axis=(0, 2)) / np.linalg.norm(ref[blk], axis=(0, 2))
            assert err.max() <= TOL["bf16"], f"segment [{b}, {e}) tokens {t0}..: output rel_F {err.max():.2e}"
    assert np.all(o[300:307] == 7.0)


@pytest.mark.parametrize("path", ["build", "prefill"])
def test_deltanet_long_segment_T(path):
    """DeltaNet (no gate) over one 6144-token segment at d = 128, built as one chain (no
    workspace) and through the cold prefill: the erase alone shrinks the transition product
    to ||T|| ~ 5e-7 with entries ~1e-8, below fp16's smallest subnormal, so the build must
    keep T's 16-bit operands scaled; T and S against the oracle."""
    W = wl.make("deltanet-16h-d128-16k", n_heads=2, lengths=[6144])
    x = workload_tensors(W)
    sb, se = dev(W.cache_begin, torch.int64), dev(W.cache_end, torch.int64)
    print(W.name, "6144 tokens", path, flush=True)
    if path == "build":
        T, S = hb.segment_build(x["k"], x["v"], x["g"], x["beta"], sb, se, gate=W.gate, delta=W.delta,
                                workspace=None)
    else:
        T, S, _ = hb.segment_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], sb, se, scale=W.scale)
    torch.cuda.synchronize()
    T0, S0 = _oracle_build(W)
    assert np.linalg.norm(T0, axis=(-2, -1)).min() > 1e-7
    eS, eT = assert_pairs_close(T.cpu().numpy(), S.cpu().numpy(), T0, S0, TOL["bf16"], W.name)
    print(f"  S {eS:.2e} T {eT:.2e}", flush=True)


def test_deltanet_d16_fp32_T():
    """d = 16, fp32 inputs, no gate: 512 tokens take T's entries to ~1e-5 (fp16 subnormal
    range for the hi/lo operand split); pairs against the oracle at the fp32 tolerance."""
    W = wl.make("deltanet-16h-d128-16k", n_heads=2, d=16, in_dtype="f32", lengths=[512, 200])
    print(W.name, "d16 fp32", flush=True)
    T, S = _gpu_build(W)
    T0, S0 = _oracle_build(W)
    eS, eT = assert_pairs_close(T, S, T0, S0, TOL["f32"], W.name)
    print(f"  S {eS:.2e} T {eT:.2e}", flush=True)


@pytest.mark.parametrize("mag", [1e5, 1e6])
@pytest.mark.parametrize("name,kw,bad", [
    ("gdn-16h-d128-32k", dict(n_heads=2, lengths=[300, 200]), 10),
    ("gdn-16h-d128-32k", dict(n_heads=2, lengths=[1500, 200]), 1200),   # in a cut segment's second piece
    ("kda-32h-d128-131k", dict(n_heads=2, lengths=[300, 200], n_req=1, n_step=1, n_layers=1), 10),
])
def test_values_beyond_fp16_range_give_non_finite_S(name, kw, bad, mag):
    """The delta-rule builds take values (GDN: v; KDA: beta * v) and states as fp16 MFMA
    operands.  An operand past fp16's range is not clamped to the largest finite fp16: it
    becomes an infinity and the S of its (segment, head) comes out non-finite, a visible
    failure rather than a wrong finite state.  So S is either non-finite or within the
    tolerance of the oracle, and at beta * |v| well past the range (here 1e6 with beta >
    0.38) it is non-finite.  T (which does not depend on v) and every other (segment, head)
    are bit for bit those of the same call without the large value."""
    W = wl.make(name, **kw)
    print(W.name, W.cache_end - W.cache_begin, "bad token", bad, "magnitude", mag, flush=True)
    x = workload_tensors(W)
    sb, se = dev(W.cache_begin, torch.int64), dev(W.cache_end, torch.int64)
    T0, S0 = hb.segment_build(x["k"], x["v"], x["g"], x["beta"], sb, se, gate=W.gate, delta=W.delta)
    v = x["v"].clone()
    v[bad, 0, :] = mag
    T1, S1 = hb.segment_build(x["k"], v, x["g"], x["beta"], sb, se, gate=W.gate, delta=W.delta)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(S0).all())
    assert torch.equal(T1, T0)
    assert torch.equal(S1[0, 1], S0[0, 1]) and torch.equal(S1[1], S0[1])
    finite = bool(torch.isfinite(S1[0, 0]).all())
    print("S finite:", finite, flush=True)
    if mag * W.beta[bad, 0] > 3e5:
        assert not finite
    if finite:
        b, e = W.cache_begin[0], W.cache_end[0]
        vb = v[b:e, 0:1].float().cpu().numpy()
        _, Sr = oracle.segment_build(W.k[b:e, 0:1], vb, W.g[b:e, 0:1], W.beta[b:e, 0:1], [0], [e - b],
                                     gate=W.gate, delta=True)
        assert rel_f(S1[0:1, 0:1].cpu().numpy(), Sr).max() <= TOL["bf16"]


@pytest.mark.parametrize("stress", [False, True])
@pytest.mark.parametrize("name,d,tol", [("gdn-16h-d128-32k", 32, "bf16"), ("gdn-tiny-f32", 32, "f32"),
                                        ("gdn-tiny-f32", 64, "f32")])
def test_gdn_d32_and_fp32_d64(name, d, tol, stress):
    """The gated delta rule at d = 32 (bf16 and fp32 inputs) and d = 64 with fp32 inputs
    (fp16 hi + lo operands): ragged, one-token and empty segments, every pair against the
    oracle and the pairs composed in order against the full recurrence."""
    W = wl.make(name, stress=stress, n_heads=2, d=d, lengths=[300, 65, 1, 0, 700])
    print(W.name, d, W.in_dtype, flush=True)
    T, S = _gpu_build(W)
    T0, S0 = _oracle_build(W)
    eS, eT = assert_pairs_close(T, S, T0, S0, TOL[tol], W.name)
    print(f"d={d} {W.in_dtype}: S {eS:.2e} T {eT}")
    Rg = torch.zeros((1, 2, d, d), device="cuda")
    hb.compose(dev(T, torch.float32), dev(S, torch.float32), dev(np.arange(5, dtype=np.int32)[None, :], torch.int32), Rg)
    torch.cuda.synchronize()
    full, _ = oracle.run(W.k, W.v, W.g, W.beta, gate=W.gate, delta=W.delta)
    assert rel_f(Rg.cpu().numpy()[0], full).max() <= TOL[tol]
