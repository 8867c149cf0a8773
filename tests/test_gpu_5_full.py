"""Full-size parity: the 32 x 1024-token gated-DeltaNet prompt and the KDA-style reuse
plan (64 requests x 256 cached segments x 30 layers), each in the launch configuration
the benchmark times, against the fp64 oracle.

The composition law ([ZH] 2.1) is checked where the pages put it: the composed state of a
whole prompt against the plain recurrence over all of its tokens, and every chain of a
request batch against the oracle's composition of the same cached pairs.
"""
import numpy as np
import pytest
import torch

import oracle
from hybrid_attention_prefill_amd import binding as hb
from hybrid_attention_prefill_amd import workloads as wl
from _util import T_FLOOR, assert_pairs_close, dev, rel_f, t_value, workload_tensors

pytestmark = pytest.mark.gpu
TOL = 5e-3


@pytest.mark.parametrize("stress", [False, True])
def test_gdn_32k_every_pair_and_the_composed_prompt(stress):
    """All 32 x 16 (segment, head) pairs of the 32k-token prompt (T cached as bf16 hi/lo
    planes, the build workspace given) against the oracle's build, then the 32 pairs
    composed in order (one chain) against the full 32768-token recurrence."""
    W = wl.make("gdn-16h-d128-32k", stress=stress)
    print(W.name, "full: every pair + composed prompt", flush=True)
    x = workload_tensors(W)
    sb, se = dev(W.cache_begin, torch.int64), dev(W.cache_end, torch.int64)
    T, S = hb.segment_build(x["k"], x["v"], x["g"], x["beta"], sb, se, gate=W.gate, delta=W.delta,
                            t_layout=hb.T_SPLIT)
    R = torch.zeros((1, W.n_heads, W.d_k, W.d_v), device="cuda")
    hb.compose(T, S, dev(W.pair_id, torch.int32), R)
    torch.cuda.synchronize()
    T0, S0 = oracle.segment_build(W.k, W.v, W.g, W.beta, W.cache_begin, W.cache_end, gate=W.gate, delta=W.delta)
    eS, eT = assert_pairs_close(t_value(T), S.cpu().numpy(), T0, S0, TOL, W.name)
    full, _ = oracle.run(W.k, W.v, W.g, W.beta, gate=W.gate, delta=W.delta)
    eR = rel_f(R.cpu().numpy()[0], full)
    print(f"  pairs: S max rel_F {eS:.2e}, T {eT}; composed prompt max rel_F {eR.max():.2e}", flush=True)
    assert eR.max() <= TOL
    if stress:   # T genuinely matters: dropping it (the naive sum) is far off
        naive = oracle.naive_sum(S.cpu().numpy(), W.pair_id)[0]
        assert rel_f(naive, full).min() > 20 * TOL


@pytest.mark.parametrize("stress", [False, True])
def test_kda_reuse_plan_full(stress):
    """The KDA-style workload as the benchmark runs it: 64 segments x 2048 tokens x 32 heads
    built (T as bf16 hi/lo planes), 30 per-layer copies of the cache, and one composition
    call over 64 requests x 30 layers = 1920 chains of 256 steps.  Checked: 8 segments'
    pairs (all heads) against the oracle's build; every request of layer 0 and sampled
    (request, layer) chains of other layers against the oracle's composition of the same
    cached pairs."""
    W = wl.make("kda-32h-d128-131k", stress=stress)
    H, d, n_seg, L = W.n_heads, W.d_k, W.n_seg, W.n_layers
    n_chain, n_step = W.pair_id.shape
    n_req = n_chain // L
    print(W.name, f"full plan: {n_chain} chains x {n_step} steps, H={H}", flush=True)
    x = workload_tensors(W)
    sb, se = dev(W.cache_begin, torch.int64), dev(W.cache_end, torch.int64)
    Tb, Sb = hb.segment_build(x["k"], x["v"], x["g"], x["beta"], sb, se, gate=W.gate, delta=W.delta,
                              t_layout=hb.T_SPLIT)
    del x
    Tc = Tb.repeat(L, 1, 1, 1)     # layer l's pairs at l * n_seg + segment
    Sc = Sb.repeat(L, 1, 1, 1)
    R = torch.zeros((n_chain, H, d, d), device="cuda")
    hb.compose(Tc, Sc, dev(W.pair_id, torch.int32), R)
    torch.cuda.synchronize()
    chains = list(range(n_req)) + [1 * n_req + 5, 7 * n_req + 63, 18 * n_req + 0, 29 * n_req + 33]
    got = R[torch.tensor(chains, device="cuda")].cpu().numpy()
    del Tc, Sc, R
    Tv, Sv = t_value(Tb), Sb.cpu().numpy()

    # the build, on 8 of the 64 segments, every head (their tokens gathered first)
    segs = np.array([0, 9, 17, 26, 38, 45, 51, 63])
    tok = np.concatenate([np.arange(W.cache_begin[s], W.cache_end[s]) for s in segs])
    lens = W.cache_end[segs] - W.cache_begin[segs]
    ends = np.cumsum(lens)
    T0, S0 = oracle.segment_build(W.k[tok], W.v[tok], W.g[tok], W.beta[tok], ends - lens, ends,
                                  gate=W.gate, delta=W.delta)
    eS, eT = assert_pairs_close(Tv[segs], Sv[segs], T0, S0, TOL, W.name)
    live = int((np.linalg.norm(T0, axis=(-2, -1)) >= T_FLOOR).sum())
    print(f"  build: S max rel_F {eS:.2e}, T {eT} ({live} of {T0.shape[0] * H} T above the floor)", flush=True)

    # the composition: layer 0, every request; then (request, layer) samples
    ids = W.pair_id[chains] - (np.array(chains) // n_req * n_seg)[:, None]
    ref = oracle.compose_gemm(Tv, Sv, ids)
    err = rel_f(got, ref)
    print(f"  compose: {len(chains)} chains x {H} heads, max rel_F {err.max():.2e}, median {np.median(err):.2e}",
          flush=True)
    assert np.all(np.isfinite(got))
    assert err.max() <= TOL
    if stress:   # every chain depends on T
        naive = oracle.naive_sum(Sv, ids[:8])
        assert rel_f(naive, ref[:8]).min() > 20 * TOL
