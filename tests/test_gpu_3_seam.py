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


def _seam_workload(name, lens, w, H, stress=False):
    """A prompt shaped like workload `name` with explicit segment lengths, seams at
    internal segments."""
    kw = dict(n_heads=H, lengths=lens, stress=stress)
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
