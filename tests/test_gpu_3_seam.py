"""hypic_seam_advance parity: seam windows stepped from the running state with
per-token outputs, then the cached pair of the rest of each segment.

References are the oracle's plain recurrence over the whole prompt (the pages:
the seam tokens are recomputed under the full prefix, so their outputs and the
final state must equal those of a full recompute).
"""
import numpy as np
import pytest
import torch

import oracle
from hybrid_attention_prefill_amd import binding as hb
from hybrid_attention_prefill_amd import workloads as wl
from _util import dev, rel_f, workload_tensors

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 5e-3}


def _seam_workload(name, lens, w, H, stress=False, **extra):
    """A prompt shaped like workload `name` with explicit segment lengths, seams at
    internal segments."""
    kw = dict(n_heads=H, lengths=lens, stress=stress, **extra)
    W = wl.make(name, **kw)
    starts = W.seg_start
    W.cache_begin = starts[:-1].copy()
    W.cache_begin[1:] += w
    W.w = w
    W.seam_start = starts[:-1].copy()[None, :]
    W.seam_start[0, 0] = -1
    return W


def _reference(W):
    """Full recurrence, with outputs only at the seam tokens (chained oracle runs)."""
    H, dv = W.n_heads, W.d_v
    k, v, g, q = (np.ascontiguousarray(a, dtype=np.float64) for a in (W.k, W.v, W.g, W.q))
    beta = np.ascontiguousarray(W.beta, dtype=np.float64)
    S = np.zeros((H, W.d_k, dv))
    outs = {}
    starts = W.seg_start
    for i in range(W.n_seg):
        a, b = int(starts[i]), int(starts[i + 1])
        if i > 0:
            S, o = oracle.run(k, v, g, beta, gate=W.gate, delta=W.delta, t0=a, t1=a + W.w, S0=S,
                              q=q, scale=W.scale)
            outs[i] = o
            a += W.w
        S, _ = oracle.run(k, v, g, beta, gate=W.gate, delta=W.delta, t0=a, t1=b, S0=S)
    return S, outs


def _gpu(W, with_pairs=True, t_layout=hb.T_SPLIT):
    x = workload_tensors(W)
    T, S = hb.segment_build(x["k"], x["v"], x["g"], x["beta"], dev(W.cache_begin, torch.int64),
                            dev(W.cache_end, torch.int64), gate=W.gate, delta=W.delta, t_layout=t_layout)
    n_step = W.n_seg
    R = torch.zeros((1, W.n_heads, W.d_k, W.d_v), device="cuda")
    out = torch.full((1, n_step, W.w, W.n_heads, W.d_v), float("nan"), device="cuda")
    hb.seam_advance(x["q"], x["k"], x["v"], x["g"], x["beta"], dev(W.seam_start, torch.int64), R, out,
                    gate=W.gate, delta=W.delta, w=W.w, scale=W.scale,
                    pair_id=dev(np.arange(n_step, dtype=np.int32)[None, :], torch.int32) if with_pairs else None,
                    T_cache=T if with_pairs else None, S_cache=S if with_pairs else None)
    torch.cuda.synchronize()
    return R.cpu().numpy()[0], out.cpu().numpy()[0]


def _check(W, R, out, S_ref, outs_ref, tol):
    assert rel_f(R, S_ref).max() <= tol, rel_f(R, S_ref).max()
    assert np.all(np.isnan(out[0]))            # no seam at the first segment: untouched
    worst = 0.0
    for i, o in outs_ref.items():
        e = rel_f(np.transpose(out[i], (1, 0, 2)), np.transpose(o, (1, 0, 2)))   # per head
        worst = max(worst, float(e.max()))
    assert worst <= tol, worst
    return worst


@pytest.mark.parametrize("w,t_layout", [(8, hb.T_SPLIT), (3, hb.T_SPLIT), (16, hb.T_SPLIT), (8, hb.T_DENSE)])
def test_seam_gdn_bf16_ragged(w, t_layout):
    W = _seam_workload("gdn-16h-d128-32k", [150, 97, 64 + w, 300, 40], w, H=2)
    print(W.name, "seam w", w, "T layout", t_layout, flush=True)
    R, out = _gpu(W, t_layout=t_layout)
    S_ref, outs_ref = _reference(W)
    _check(W, R, out, S_ref, outs_ref, TOL["bf16"])


def test_seam_gdn_bf16_stress():
    W = _seam_workload("gdn-16h-d128-32k", [512, 530, 600, 520], 8, H=2, stress=True)
    R, out = _gpu(W)
    S_ref, outs_ref = _reference(W)
    _check(W, R, out, S_ref, outs_ref, TOL["bf16"])


@pytest.mark.parametrize("stress,t_layout", [(False, hb.T_SPLIT), (True, hb.T_SPLIT), (True, hb.T_DENSE)])
def test_seam_gdn_fp32_d16(stress, t_layout):
    W = _seam_workload("gdn-tiny-f32", [64, 40, 77], 8, H=1, stress=stress)
    print(W.name, "fp32 seam", stress, t_layout, flush=True)
    R, out = _gpu(W, t_layout=t_layout)
    S_ref, outs_ref = _reference(W)
    _check(W, R, out, S_ref, outs_ref, TOL["f32"])


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64), (64, 16)])
@pytest.mark.parametrize("lens", [[150, 97, 72, 300, 40], [40 + (7 * i) % 23 for i in range(48)]])
def test_seam_rectangular_state(lens, dk, dv):
    """d_k != d_v: a wider state (64 x 128) advances in two blocks of 64 columns through one
    workspace, a narrower one (128 x 64, 64 x 16) in one pass whose column blocks end at its
    last column; a short prompt (plain chain) and a 48-segment one (blocked scan), against the
    full recurrence: final state and every window's outputs."""
    W = _seam_workload("gdn-16h-d128-32k", lens, 8, H=2, d=dk)
    rng = np.random.default_rng(64128 + len(lens) + dk + dv)
    W.v = wl.round_bf16(rng.standard_normal((W.n_tokens, 2, dv)))
    W.d_v = dv
    print(W.name, "rectangular seam", len(lens), "segments", flush=True)
    R, out = _gpu(W)
    S_ref, outs_ref = _reference(W)
    worst = _check(W, R, out, S_ref, outs_ref, TOL["bf16"])
    print(f"  outputs rel_F max {worst:.2e}", flush=True)


def test_seam_only_without_pairs():
    """pair_id NULL: only the seam windows advance the state."""
    W = _seam_workload("gdn-16h-d128-32k", [40, 30, 50], 8, H=2)
    R, out = _gpu(W, with_pairs=False)
    S = np.zeros((2, 128, 128))
    for i in (1, 2):
        a = int(W.seg_start[i])
        S, o = oracle.run(W.k, W.v, W.g, W.beta, gate=W.gate, delta=True, t0=a, t1=a + 8, S0=S, q=W.q,
                          scale=W.scale)
        e = rel_f(np.transpose(out[i], (1, 0, 2)), np.transpose(o, (1, 0, 2)))
        assert e.max() <= TOL["bf16"]
    assert rel_f(R, S).max() <= TOL["bf16"]


def test_gdn_100k_prompt_full():
    """The 100k-token prompt (128 lognormal segments, 16 heads, d=128, w=8) in the
    benchmark's launch configuration: final state and all 127 windows' outputs."""
    W = wl.make("gdn-16h-d128-100k-seam")
    print(W.name, flush=True)
    R, out = _gpu(W)
    S_ref, outs_ref = _reference(W)
    worst = _check(W, R, out, S_ref, outs_ref, TOL["bf16"])
    print(f"100k prompt: final state rel_F {rel_f(R, S_ref).max():.2e}, worst window output {worst:.2e}")


# ---- long chains: the call runs as a blocked scan (blocks of steps at once, block
# aggregates composed in order, window outputs read out from the block entry states)

def _short_lengths(rng, n, w, lo=20, hi=60):
    return list(int(x) for x in rng.integers(lo, hi, size=n) + w)


@pytest.mark.parametrize("stress,t_layout", [(False, hb.T_SPLIT), (True, hb.T_SPLIT), (True, hb.T_DENSE)])
def test_seam_scan_many_steps(stress, t_layout):
    rng = np.random.default_rng(11)
    W = _seam_workload("gdn-16h-d128-32k", _short_lengths(rng, 40, 8), 8, H=2, stress=stress)
    print(W.name, "scan, 40 steps, stress", stress, "T layout", t_layout, flush=True)
    R, out = _gpu(W, t_layout=t_layout)
    S_ref, outs_ref = _reference(W)
    _check(W, R, out, S_ref, outs_ref, TOL["bf16"])


@pytest.mark.parametrize("stress", [False, True])
def test_seam_scan_fp32_d16(stress):
    rng = np.random.default_rng(12)
    W = _seam_workload("gdn-tiny-f32", _short_lengths(rng, 26, 8, 10, 40), 8, H=1, stress=stress)
    print(W.name, "fp32 scan, 26 steps, stress", stress, flush=True)
    R, out = _gpu(W)
    S_ref, outs_ref = _reference(W)
    _check(W, R, out, S_ref, outs_ref, TOL["f32"])


def test_seam_scan_without_pairs():
    rng = np.random.default_rng(13)
    W = _seam_workload("gdn-16h-d128-32k", _short_lengths(rng, 24, 8, 8, 12), 8, H=2, stress=True)
    R, out = _gpu(W, with_pairs=False)
    S = np.zeros((2, 128, 128))
    for i in range(1, W.n_seg):
        a = int(W.seg_start[i])
        S, o = oracle.run(W.k, W.v, W.g, W.beta, gate=W.gate, delta=True, t0=a, t1=a + 8, S0=S, q=W.q,
                          scale=W.scale)
        e = rel_f(np.transpose(out[i], (1, 0, 2)), np.transpose(o, (1, 0, 2)))
        assert e.max() <= TOL["bf16"], (i, e.max())
    assert rel_f(R, S).max() <= TOL["bf16"]


def test_long_chain_composition_through_the_scan():
    """One long chain of compositions without windows (every seam_start -1) through
    hypic_seam_advance, which runs it as a blocked scan: the 32 x 1024 stress pairs at 16 heads
    composed along 128 steps (each pair four times, out of order) equal the serial
    hypic_compose and the fp64 composition of the same pairs."""
    W = wl.make("gdn-16h-d128-32k", stress=True)
    x = workload_tensors(W)
    T, S = hb.segment_build(x["k"], x["v"], x["g"], x["beta"], dev(W.cache_begin, torch.int64),
                            dev(W.cache_end, torch.int64), gate=W.gate, delta=W.delta, t_layout=hb.T_SPLIT)
    rng = np.random.default_rng(17)
    ids = np.concatenate([rng.permutation(32) for _ in range(4)]).astype(np.int32)[None, :]
    pid = dev(ids, torch.int32)
    H, d, n_step = W.n_heads, 128, ids.shape[1]
    R_ser = torch.zeros((1, H, d, d), device="cuda")
    hb.compose(T, S, pid, R_ser)
    R_scan = torch.zeros_like(R_ser)
    out = torch.zeros((1, n_step, 8, H, d), device="cuda")
    ws = torch.empty(hb.seam_workspace_bytes(H, d, d, 1, n_step, 8), dtype=torch.uint8, device="cuda")
    hb.seam_advance(x["k"], x["k"], x["v"], x["g"], x["beta"], dev(np.full((1, n_step), -1, np.int64), torch.int64),
                    R_scan, out, gate=W.gate, delta=W.delta, w=8, scale=1.0, pair_id=pid, T_cache=T, S_cache=S,
                    workspace=ws)
    torch.cuda.synchronize()
    T0, S0 = oracle.segment_build(W.k, W.v, W.g, W.beta, W.cache_begin, W.cache_end, gate=W.gate, delta=W.delta)
    ref = oracle.compose(T0, S0, ids)[0]
    e_scan = rel_f(R_scan.cpu().numpy()[0], ref).max()
    e_ser = rel_f(R_ser.cpu().numpy()[0], ref).max()
    print(f"128-step chain: scan {e_scan:.2e}, serial {e_ser:.2e}")
    assert e_scan <= TOL["bf16"] and e_ser <= TOL["bf16"]
    assert np.all(out.cpu().numpy() == 0)   # no window: no output row is written


@pytest.mark.parametrize("d", [64, 128])
def test_seam_scan_two_chains_mixed_plan(d):
    """Two chains from nonzero states; chain 1 skips some windows and some pairs and
    reuses segments out of order.  Reference: oracle windows and fp64 composition with
    the oracle's own pairs, step by step."""
    rng = np.random.default_rng(14 + d)
    H, w, n = 2, 8, 24
    W = _seam_workload("gdn-16h-d128-32k", _short_lengths(rng, n, w), w, H=H, stress=True, d=d)
    starts = W.seg_start
    seam = np.stack([starts[:-1], starts[:-1]]).astype(np.int64)
    seam[:, 0] = -1
    seam[1, rng.choice(np.arange(1, n), 6, replace=False)] = -1
    pid = np.stack([np.arange(n), rng.permutation(n)]).astype(np.int32)
    pid[1, rng.choice(n, 5, replace=False)] = -1
    R0 = rng.standard_normal((2, H, d, d)) * 0.3
    x = workload_tensors(W)
    T, S = hb.segment_build(x["k"], x["v"], x["g"], x["beta"], dev(W.cache_begin, torch.int64),
                            dev(W.cache_end, torch.int64), gate=W.gate, delta=W.delta, t_layout=hb.T_SPLIT)
    R = dev(R0, torch.float32)
    out = torch.full((2, n, w, H, d), float("nan"), device="cuda")
    hb.seam_advance(x["q"], x["k"], x["v"], x["g"], x["beta"], dev(seam, torch.int64), R, out,
                    gate=W.gate, delta=W.delta, w=w, scale=W.scale, pair_id=dev(pid, torch.int32),
                    T_cache=T, S_cache=S)
    torch.cuda.synchronize()
    R, out = R.cpu().numpy(), out.cpu().numpy()
    T0, S0 = oracle.segment_build(W.k, W.v, W.g, W.beta, W.cache_begin, W.cache_end, gate=W.gate, delta=True)
    for c in range(2):
        Sr = R0[c].copy()
        for j in range(n):
            if seam[c, j] >= 0:
                a = int(seam[c, j])
                Sr, o = oracle.run(W.k, W.v, W.g, W.beta, gate=W.gate, delta=True, t0=a, t1=a + w, S0=Sr,
                                   q=W.q, scale=W.scale)
                e = rel_f(np.transpose(out[c, j], (1, 0, 2)), np.transpose(o, (1, 0, 2)))
                assert e.max() <= TOL["bf16"], (c, j, e.max())
            else:
                assert np.all(np.isnan(out[c, j])), (c, j)
            if pid[c, j] >= 0:
                Sr = T0[pid[c, j]] @ Sr + S0[pid[c, j]]
        assert rel_f(R[c], Sr).max() <= TOL["bf16"], (c, rel_f(R[c], Sr).max())


def test_seam_scan_blocks_longer_than_the_id_ring():
    """32 chains x 600 steps, 4 heads, d = 64, w = 2: the call runs 2 blocks of 300 steps
    (longer than the kernel's 256-step id ring, so the ring refills inside a block).
    Every chain starts from its own state and reuses the same segments; all outputs and
    final states against the oracle (fp64 composition of the oracle's own pairs)."""
    rng = np.random.default_rng(21)
    H, d, w, n, n_chain = 4, 64, 2, 600, 32
    W = _seam_workload("gdn-16h-d128-32k", [6] * n, w, H=H, stress=True, d=d)
    starts = W.seg_start
    seam = np.tile(starts[:-1], (n_chain, 1)).astype(np.int64)
    seam[:, 0] = -1
    pid = np.tile(np.arange(n, dtype=np.int32), (n_chain, 1))
    R0 = rng.standard_normal((n_chain, H, d, d)) * 0.3
    x = workload_tensors(W)
    T, S = hb.segment_build(x["k"], x["v"], x["g"], x["beta"], dev(W.cache_begin, torch.int64),
                            dev(W.cache_end, torch.int64), gate=W.gate, delta=W.delta, t_layout=hb.T_SPLIT)
    R = dev(R0, torch.float32)
    out = torch.full((n_chain, n, w, H, d), float("nan"), device="cuda")
    print("600-step chains", flush=True)
    hb.seam_advance(x["q"], x["k"], x["v"], x["g"], x["beta"], dev(seam, torch.int64), R, out,
                    gate=W.gate, delta=W.delta, w=w, scale=W.scale, pair_id=dev(pid, torch.int32),
                    T_cache=T, S_cache=S)
    torch.cuda.synchronize()
    R, out = R.cpu().numpy(), out.cpu().numpy()
    T0, S0 = oracle.segment_build(W.k, W.v, W.g, W.beta, W.cache_begin, W.cache_end, gate=W.gate, delta=True)
    Sr = R0.copy()                                   # [chain][head][d][d], all chains at once
    worst = 0.0
    for j in range(n):
        if j > 0:
            a = int(starts[j])
            for c in range(n_chain):
                Sr[c], o = oracle.run(W.k, W.v, W.g, W.beta, gate=W.gate, delta=True, t0=a, t1=a + w, S0=Sr[c],
                                      q=W.q, scale=W.scale)
                worst = max(worst, float(rel_f(np.transpose(out[c, j], (1, 0, 2)), np.transpose(o, (1, 0, 2))).max()))
        Sr = T0[j][None] @ Sr + S0[j][None]
    assert worst <= TOL["bf16"], worst
    assert np.all(np.isnan(out[:, 0]))
    assert rel_f(R, Sr).max() <= TOL["bf16"], rel_f(R, Sr).max()
