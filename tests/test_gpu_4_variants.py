"""The other transition families against the fp64 oracle: GLA-style per-channel
gates without the erase (diagonal T, cached as its diagonal), Mamba2-style token
gates without the erase (scalar T) and DeltaNet (erase without a gate).

Tolerances as for the other builds: relative Frobenius error per (segment, head)
<= 1e-4 for fp32 inputs and <= 5e-3 for bf16 inputs.
"""
import numpy as np
import pytest
import torch

import oracle
from hybrid_attention_prefill_amd import binding as hb
from hybrid_attention_prefill_amd import workloads as wl
from _util import assert_pairs_close, dev, rel_f, t_value, workload_tensors

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 5e-3}


def _build(W, t_layout, begin=None, end=None):
    x = workload_tensors(W)
    b = W.cache_begin if begin is None else begin
    e = W.cache_end if end is None else end
    T, S = hb.segment_build(x["k"], x["v"], x["g"], x["beta"], dev(b, torch.int64), dev(e, torch.int64),
                            gate=W.gate, delta=W.delta, t_layout=t_layout)
    torch.cuda.synchronize()
    return T, S.cpu().numpy()


def _dense(T, t_layout, d):
    """A T cache of any layout as float64 [..., d, d]."""
    if t_layout == hb.T_DIAG:
        t = T.double().cpu().numpy()
        return t[..., :, None] * np.eye(d)
    if t_layout == hb.T_SCALAR:
        return T.double().cpu().numpy()[..., None, None] * np.eye(d)
    return t_value(T, d)


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("t_layout", [hb.T_DIAG, hb.T_DENSE, hb.T_SPLIT])
def test_gla_build(t_layout, d, in_dtype):
    """Per-channel gate, no erase: chunks, ragged tails, one token, an empty range."""
    W = wl.make("gla-16h-d128-16k", n_heads=3, d=d, lengths=[300, 64, 1, 129], in_dtype=in_dtype)
    begin = np.concatenate([W.cache_begin, [7]])
    end = np.concatenate([W.cache_end, [7]])
    print(W.name, d, in_dtype, t_layout, flush=True)
    T, S = _build(W, t_layout, begin, end)
    T0, S0 = oracle.segment_build(W.k, W.v, W.g, W.beta, begin, end, gate=W.gate, delta=False)
    Td = _dense(T, t_layout, d)
    assert_pairs_close(Td, S, T0, S0, TOL[in_dtype], W.name)
    if t_layout == hb.T_DENSE:
        off = Td * (1 - np.eye(d))
        assert np.all(off == 0)                      # diagonal T has exact zeros off the diagonal
    assert np.array_equal(Td[-1], np.broadcast_to(np.eye(d), Td[-1].shape))
    assert np.all(S[-1] == 0)


@pytest.mark.parametrize("stress", [False, True])
def test_gla_full_size_compose_matches_full(stress):
    """16 heads x 16 x 1024 tokens at d=128 (the workload's full shape): the diagonal
    pairs composed in order equal the full recurrence; under stress the naive sum does not."""
    W = wl.make("gla-16h-d128-16k", stress=stress)
    print(W.name, "full", flush=True)
    T, S = _build(W, hb.T_DIAG)
    assert tuple(T.shape) == (16, 16, 128) and T.dtype == torch.float32
    Rg = torch.zeros((1, 16, 128, 128), device="cuda")
    hb.compose(T, dev(S, torch.float32), dev(W.pair_id, torch.int32), Rg)
    torch.cuda.synchronize()
    full, _ = oracle.run(W.k, W.v, W.g, None, gate=W.gate, delta=False)
    assert rel_f(Rg.cpu().numpy()[0], full).max() <= TOL["bf16"]
    rng = np.random.default_rng(2)
    for s, h in zip(rng.integers(0, 16, 3), rng.integers(0, 16, 3)):
        b, e = W.cache_begin[s], W.cache_end[s]
        T0, S0 = oracle.segment_build(W.k[b:e, h:h + 1], W.v[b:e, h:h + 1], W.g[b:e, h:h + 1], None,
                                      [0], [e - b], gate=W.gate, delta=False)
        assert_pairs_close(_dense(T[s:s + 1, h:h + 1], hb.T_DIAG, 128), S[s:s + 1, h:h + 1], T0, S0,
                           TOL["bf16"], f"seg {s} head {h}")
    if stress:
        naive = oracle.naive_sum(S, W.pair_id)[0]
        assert rel_f(naive, full).min() > 20 * TOL["bf16"]


@pytest.mark.parametrize("dk,dv", [(16, 16), (64, 64), (128, 128), (128, 64), (32, 128)])
def test_compose_diag_T(dk, dv):
    """Elementwise composition with diagonal T: row r of the state scales by t[r]."""
    H, n_pair, n_chain, n_step = 5, 7, 3, 9
    rng = np.random.default_rng(dk + dv)
    t = rng.uniform(0.3, 1.0, size=(n_pair, H, dk)).astype(np.float32)
    S = rng.standard_normal((n_pair, H, dk, dv)).astype(np.float32)
    ids = rng.integers(-1, n_pair, size=(n_chain, n_step)).astype(np.int32)
    ids[1, 2] = n_pair + 4                            # out of range: skipped
    R0 = rng.standard_normal((n_chain, H, dk, dv)).astype(np.float32)
    Td = t.astype(np.float64)[..., :, None] * np.eye(dk)
    ref = oracle.compose(Td, S, np.where(ids >= n_pair, -1, ids), R0)
    Rg = dev(R0, torch.float32)
    hb.compose(dev(t, torch.float32), dev(S, torch.float32), dev(ids, torch.int32), Rg, t_layout=hb.T_DIAG)
    torch.cuda.synchronize()
    assert rel_f(Rg.cpu().numpy(), ref).max() < 1e-6


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("t_layout", [hb.T_SCALAR, hb.T_DENSE])
def test_mamba2_build_and_compose(t_layout, in_dtype):
    """Token scalar gate, no erase (d=64): pairs with ragged tails, then the ordered
    composition against the full recurrence."""
    W = wl.make("mamba2-16h-d64-16k", n_heads=4, lengths=[1024, 77, 1, 640], in_dtype=in_dtype)
    print(W.name, in_dtype, t_layout, flush=True)
    T, S = _build(W, t_layout)
    T0, S0 = oracle.segment_build(W.k, W.v, W.g, None, W.cache_begin, W.cache_end, gate=W.gate, delta=False)
    assert_pairs_close(_dense(T, t_layout, 64), S, T0, S0, TOL[in_dtype], W.name)
    Rg = torch.zeros((1, 4, 64, 64), device="cuda")
    hb.compose(T, dev(S, torch.float32), dev(W.pair_id, torch.int32), Rg, t_layout=t_layout)
    torch.cuda.synchronize()
    full, _ = oracle.run(W.k, W.v, W.g, None, gate=W.gate, delta=False)
    assert rel_f(Rg.cpu().numpy()[0], full).max() <= TOL[in_dtype]


@pytest.mark.parametrize("stress", [False, True])
def test_deltanet_build_and_compose(stress):
    """Erase without a gate (g = 0), d=128, bf16: T is a product of I - b k k^T, which
    stays O(1), so the composition exercises T at full weight."""
    W = wl.make("deltanet-16h-d128-16k", stress=stress, n_heads=2, lengths=[1024, 300, 65, 1])
    print(W.name, flush=True)
    T, S = _build(W, hb.T_DENSE)
    T = T.cpu().numpy()
    T0, S0 = oracle.segment_build(W.k, W.v, W.g, W.beta, W.cache_begin, W.cache_end, gate=W.gate, delta=True)
    assert_pairs_close(T, S, T0, S0, TOL["bf16"], W.name)
    Rg = torch.zeros((1, 2, 128, 128), device="cuda")
    hb.compose(dev(T, torch.float32), dev(S, torch.float32), dev(W.pair_id, torch.int32), Rg)
    torch.cuda.synchronize()
    full, _ = oracle.run(W.k, W.v, W.g, W.beta, gate=W.gate, delta=True)
    assert rel_f(Rg.cpu().numpy()[0], full).max() <= TOL["bf16"]
    naive = oracle.naive_sum(S, W.pair_id)[0]
    assert rel_f(naive, full).min() > 10 * TOL["bf16"]


@pytest.mark.parametrize("stress", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_kda_gate_first_ragged(d, stress):
    """KDA with the gate applied before the erase, (I - b k k^T) diag(a_t), and log-gates
    spread widely over the channels (g = -softplus(2 z)): several chunks, ragged tails, one
    token, an empty range.  Without stress the gate-after-erase states of the same tokens
    differ from these (by more than three times the tolerance at the median), and the
    GPU's states are checked to be far from them, so the order is tested."""
    W = wl.make("kda-32h-d128-131k", gate_first=True, gate_sigma=2.0, stress=stress, n_heads=2, d=d,
                lengths=[256, 100, 33, 1], n_req=1, n_step=1, n_layers=1)
    assert W.delta == 2
    begin = np.concatenate([W.cache_begin, [3]])
    end = np.concatenate([W.cache_end, [3]])
    print(W.name, d, flush=True)
    T, S = _build(W, hb.T_DENSE, begin, end)
    T = T.cpu().numpy()
    T0, S0 = oracle.segment_build(W.k, W.v, W.g, W.beta, begin, end, gate=W.gate, delta=2)
    assert_pairs_close(T, S, T0, S0, TOL["bf16"], W.name)
    assert np.array_equal(T[-1], np.broadcast_to(np.eye(d, dtype=np.float32), T[-1].shape)) and np.all(S[-1] == 0)
    if not stress:
        _, S1 = oracle.segment_build(W.k, W.v, W.g, W.beta, begin, end, gate=W.gate, delta=1)
        assert np.median(rel_f(S1[:3], S0[:3])) > 3 * TOL["bf16"]
        assert rel_f(S[:3], S1[:3]).max() > 2 * TOL["bf16"]


def test_kda_gate_first_split_compose_matches_full():
    """Gate-first KDA pairs cached with SPLIT T and composed in order equal the full recurrence."""
    W = wl.make("kda-32h-d128-131k", gate_first=True, gate_sigma=2.0, stress=True, n_heads=2, n_seg=4,
                seg_len=300, n_req=1, n_step=1, n_layers=1)
    print(W.name, "split compose", flush=True)
    T, S = _build(W, hb.T_SPLIT)
    Rg = torch.zeros((1, 2, 128, 128), device="cuda")
    hb.compose(T, dev(S, torch.float32), dev(np.arange(4, dtype=np.int32)[None, :], torch.int32), Rg)
    torch.cuda.synchronize()
    full, _ = oracle.run(W.k, W.v, W.g, W.beta, gate=W.gate, delta=2)
    assert rel_f(Rg.cpu().numpy()[0], full).max() <= TOL["bf16"]
    naive = oracle.naive_sum(S, np.arange(4)[None, :])[0]
    assert rel_f(naive, full).min() > 20 * TOL["bf16"]


# ---- builds without the erase cut into pieces (build workspace): up to 8 runs of whole
# chunks per segment built in parallel and composed elementwise

@pytest.mark.parametrize("name,in_dtype,t_layout", [
    ("retnet-8h-d64", "bf16", hb.T_SCALAR), ("retnet-8h-d64", "bf16", hb.T_SPLIT),
    ("mamba2-16h-d64-16k", "f32", hb.T_SCALAR), ("mamba2-16h-d64-16k", "bf16", hb.T_DENSE),
    ("gla-16h-d128-16k", "bf16", hb.T_DIAG), ("gla-16h-d128-16k", "f32", hb.T_SPLIT)])
def test_decay_build_in_pieces(name, in_dtype, t_layout):
    """21, 1, 1, 10 and 4 chunks (ragged tails, one token) and an empty range, built in
    pieces and as one chain, both against the oracle; a segment's pair is bit-identical
    whether it is built alone or in the batch."""
    kw = {} if name.startswith("retnet") else {"in_dtype": in_dtype}
    W = wl.make(name, n_heads=2, lengths=[1300, 64, 1, 577, 200], **kw)
    begin = np.concatenate([W.cache_begin, [7]])
    end = np.concatenate([W.cache_end, [7]])
    d = W.d_k
    x = workload_tensors(W)
    need = hb.build_workspace_bytes(2, d, d, len(begin), W.n_tokens, gate=W.gate, delta=False,
                                    in_dtype=hb.BF16 if W.in_dtype == "bf16" else hb.F32)
    assert need > 0
    ws = torch.empty(need, device="cuda", dtype=torch.uint8)
    print(W.name, in_dtype, t_layout, need, flush=True)

    def build(b, e, workspace):
        T, S = hb.segment_build(x["k"], x["v"], x["g"], x["beta"], dev(b, torch.int64), dev(e, torch.int64),
                                gate=W.gate, delta=False, t_layout=t_layout, workspace=workspace)
        torch.cuda.synchronize()
        return T, S.cpu().numpy()

    T0, S0 = oracle.segment_build(W.k, W.v, W.g, W.beta, begin, end, gate=W.gate, delta=False)
    for workspace in (ws, None):
        T, S = build(begin, end, workspace)
        assert_pairs_close(_dense(T, t_layout, d), S, T0, S0, TOL[W.in_dtype], f"{W.name} ws={workspace is not None}")
        assert np.all(S[-1] == 0)
    Tb, Sb = build(begin, end, ws)
    Ta, Sa = build(begin[3:4], end[3:4], ws)
    assert np.array_equal(Sa[0], Sb[3])
    assert torch.equal(Ta[0], Tb[3])


@pytest.mark.parametrize("ws", ["auto", None])
@pytest.mark.parametrize("dk,dv", [(16, 64), (128, 32), (64, 128)])
@pytest.mark.parametrize("gate", [hb.GATE_HEAD, hb.GATE_TOKEN, hb.GATE_DIAG])
def test_decay_build_rectangular_state(gate, dk, dv, ws):
    """d_k != d_v without the erase (RetNet-, Mamba2- and GLA-style gates), bf16 inputs:
    every pair against the oracle, with and without the pieces workspace, then the pairs
    composed in order (scalar or diagonal T) against the full recurrence over the segments."""
    print(f"rectangular gate={gate} dk={dk} dv={dv} ws={ws}", flush=True)
    rng = np.random.default_rng(1000 * gate + dk + dv)
    H = 2
    lens = np.array([600, 333, 1, 0, 366])
    N = int(lens.sum())
    begin = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    end = begin + lens
    kx = rng.standard_normal((N, H, dk))
    k = wl.round_bf16(kx / np.linalg.norm(kx, axis=-1, keepdims=True))
    v = wl.round_bf16(rng.standard_normal((N, H, dv)))
    beta = None
    if gate == hb.GATE_HEAD:
        g = np.log1p(-np.exp2(-5.0 - np.arange(H))).astype(np.float32)
        gt = torch.float32
        t_layout = hb.T_SCALAR
    elif gate == hb.GATE_TOKEN:
        g = wl.round_bf16(-0.1 * np.logaddexp(0.0, rng.standard_normal((N, H))))
        gt = torch.bfloat16
        t_layout = hb.T_SCALAR
    else:
        g = wl.round_bf16(-np.logaddexp(0.0, rng.standard_normal((N, H, dk))) / 16.0)
        gt = torch.bfloat16
        t_layout = hb.T_DIAG
    kd, vd, gd = dev(k, torch.bfloat16), dev(v, torch.bfloat16), dev(g, gt)
    sb, se = dev(begin, torch.int64), dev(end, torch.int64)
    T, S = hb.segment_build(kd, vd, gd, None, sb, se, gate=gate, delta=0, t_layout=t_layout, workspace=ws)
    torch.cuda.synchronize()
    T0, S0 = oracle.segment_build(k, v, g, None, begin, end, gate=gate, delta=0)
    Sg = S.cpu().numpy()
    assert np.all(np.isfinite(Sg))
    assert rel_f(Sg, S0).max() <= TOL["bf16"]
    assert rel_f(_dense(T, t_layout, dk), T0).max() <= TOL["bf16"]
    R = torch.zeros((1, H, dk, dv), device="cuda")
    hb.compose(T, S, dev(np.arange(len(lens), dtype=np.int32)[None, :], torch.int32), R)
    torch.cuda.synchronize()
    full, _ = oracle.run(k, v, g, None, gate=gate, delta=0)
    assert rel_f(R.cpu().numpy()[0], full).max() <= TOL["bf16"]


@pytest.mark.parametrize("family,dk,dv,in_dtype,delta", [
    ("gdn", 64, 128, "bf16", 1), ("gdn", 32, 128, "bf16", 1), ("gdn", 16, 32, "f32", 1),
    ("kda", 64, 128, "bf16", 1), ("kda", 64, 128, "bf16", 2),
    ("gdn", 128, 64, "bf16", 1), ("gdn", 32, 16, "f32", 1), ("kda", 128, 32, "bf16", 1), ("kda", 128, 64, "bf16", 2),
    ("kda", 32, 32, "bf16", 1), ("kda", 16, 16, "bf16", 2), ("kda", 32, 128, "bf16", 1), ("kda", 16, 64, "bf16", 2)])
def test_delta_build_rectangular_state(family, dk, dv, in_dtype, delta):
    """d_k != d_v with the delta rule (its columns evolve independently): a multiple of d_k
    is built as d_v / d_k blocks of d_k columns, a narrower state in one launch with the
    missing value columns read as zeros.  Every pair against the oracle; each column block
    bit-identical to a square build of the same value columns; the pairs composed in order
    against the full recurrence."""
    print(f"rectangular delta family={family} dk={dk} dv={dv} in={in_dtype} delta={delta}", flush=True)
    rng = np.random.default_rng(7000 + 100 * dk + dv + delta)
    H = 2
    lens = np.array([600, 333, 1, 0, 366])
    N = int(lens.sum())
    begin = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    end = begin + lens
    rnd = wl.round_bf16 if in_dtype == "bf16" else (lambda a: a.astype(np.float32))
    tt = torch.bfloat16 if in_dtype == "bf16" else torch.float32
    kx = rng.standard_normal((N, H, dk))
    k = rnd(kx / np.linalg.norm(kx, axis=-1, keepdims=True))
    v = rnd(rng.standard_normal((N, H, dv)))
    beta = rnd(1.0 / (1.0 + np.exp(-rng.standard_normal((N, H)))))
    if family == "gdn":
        gate = hb.GATE_TOKEN
        g = rnd(-0.1 * np.logaddexp(0.0, rng.standard_normal((N, H))))
    else:
        gate = hb.GATE_DIAG
        g = rnd(-np.logaddexp(0.0, rng.standard_normal((N, H, dk))) / 16.0)
    kd, gd, bd = dev(k, tt), dev(g, tt), dev(beta, tt)
    sb, se = dev(begin, torch.int64), dev(end, torch.int64)
    T, S = hb.segment_build(kd, dev(v, tt), gd, bd, sb, se, gate=gate, delta=delta, t_layout=hb.T_SPLIT)
    torch.cuda.synchronize()
    T0, S0 = oracle.segment_build(k, v, g, beta, begin, end, gate=gate, delta=delta)
    Sg = S.cpu().numpy()
    eS, eT = assert_pairs_close(t_value(T, dk), Sg, T0, S0, TOL[in_dtype], f"{family} {dk}x{dv}")
    print(f"  S rel_F max {eS:.2e}, T rel_F max {eT}", flush=True)
    for j in range(dv // dk):   # each column block as a square build of the same columns
        Tj, Sj = hb.segment_build(kd, dev(np.ascontiguousarray(v[:, :, j * dk:(j + 1) * dk]), tt), gd, bd, sb, se,
                                  gate=gate, delta=delta, t_layout=hb.T_SPLIT)
        torch.cuda.synchronize()
        assert np.array_equal(Sj.cpu().numpy(), Sg[..., j * dk:(j + 1) * dk]), f"column block {j}"
        assert torch.equal(Tj, T)
    R = torch.zeros((1, H, dk, dv), device="cuda")
    hb.compose(T, S, dev(np.arange(len(lens), dtype=np.int32)[None, :], torch.int32), R)
    torch.cuda.synchronize()
    full, _ = oracle.run(k, v, g, beta, gate=gate, delta=delta)
    eR = rel_f(R.cpu().numpy()[0], full).max()
    assert eR <= TOL[in_dtype], f"composed state rel_F {eR:.3e}"
