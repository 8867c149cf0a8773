"""hypic_seam_advance_noalloc (the library's static device scratch instead of a caller
workspace) against hypic_seam_advance (caller workspace) on the same inputs: two calls in a
row, the second smaller than the first, and a call too large for the scratch."""
import numpy as np
import pytest
import torch

from hybrid_attention_prefill_amd import binding as hb
from hybrid_attention_prefill_amd import workloads as wl
from _util import dev, workload_tensors

pytestmark = pytest.mark.gpu


def _case(lengths, heads, n_cached_pairs):
    """A prompt of segments with seam windows at every internal segment, its pairs built."""
    W = wl.make("gdn-16h-d128-100k-seam", n_heads=heads, n_seg=len(lengths), total=int(sum(lengths)),
                minimum=min(lengths), median=int(np.median(lengths)))
    x = workload_tensors(W)
    T, S = hb.segment_build(x["k"], x["v"], x["g"], x["beta"], dev(W.cache_begin, torch.int64),
                            dev(W.cache_end, torch.int64), gate=W.gate, delta=W.delta, t_layout=hb.T_SPLIT)
    return W, x, T, S


def _both(W, x, T, S, R0):
    seam = dev(W.seam_start, torch.int64)
    ids = dev(W.pair_id, torch.int32)
    out_shape = (1, W.n_seg, W.w, W.n_heads, W.d_v)
    Ra, oa = R0.clone(), torch.full(out_shape, 5.0, device="cuda")
    hb.seam_advance(x["q"], x["k"], x["v"], x["g"], x["beta"], seam, Ra, oa, gate=W.gate, delta=W.delta, w=W.w,
                    scale=W.scale, pair_id=ids, T_cache=T, S_cache=S)
    Rb, ob = R0.clone(), torch.full(out_shape, 5.0, device="cuda")
    hb.seam_advance_noalloc(x["q"], x["k"], x["v"], x["g"], x["beta"], seam, Rb, ob, gate=W.gate, delta=W.delta,
                            w=W.w, scale=W.scale, pair_id=ids, T_cache=T, S_cache=S)
    torch.cuda.synchronize()
    return (Ra, oa), (Rb, ob)


def test_noalloc_matches_workspace_call_twice():
    """First a 48-step chain at 8 heads (run as a blocked scan: window records, readouts,
    block aggregates and the trail all in the scratch), then a 6-step chain at 2 heads (the
    plain chain): bit-identical to the calls with a caller workspace."""
    first = _case([600] * 48, 8, 48)
    need = hb.seam_workspace_bytes(8, 128, 128, 1, 48, 8)
    print(f"no-alloc call 1: 48 steps x 8 heads, {need / 2**20:.1f} MiB of scratch", flush=True)
    assert 0 < need <= hb.NOALLOC_SCRATCH_BYTES
    R0 = torch.randn((1, 8, 128, 128), device="cuda") * 0.1
    (Ra, oa), (Rb, ob) = _both(*first, R0)
    assert torch.equal(Ra, Rb) and torch.equal(oa, ob)
    second = _case([520] * 6, 2, 6)
    print("no-alloc call 2: 6 steps x 2 heads", flush=True)
    R0 = torch.zeros((1, 2, 128, 128), device="cuda")
    (Ra, oa), (Rb, ob) = _both(*second, R0)
    assert torch.equal(Ra, Rb) and torch.equal(oa, ob)
    assert bool((ob[0, 0] == 5.0).all())   # the first segment has no seam window: its rows untouched


def test_noalloc_rejects_calls_beyond_the_scratch():
    """A plan whose workspace exceeds the static scratch is refused before any launch."""
    H, n_step = 16, 256
    need = hb.seam_workspace_bytes(H, 128, 128, 1, n_step, 8)
    assert need > hb.NOALLOC_SCRATCH_BYTES
    n_tok = 64
    k = torch.zeros((n_tok, H, 128), device="cuda", dtype=torch.bfloat16)
    g = torch.zeros((n_tok, H), device="cuda", dtype=torch.bfloat16)
    seam = torch.full((1, n_step), -1, device="cuda", dtype=torch.int64)
    R = torch.full((1, H, 128, 128), 3.0, device="cuda")
    out = torch.full((1, n_step, 8, H, 128), 3.0, device="cuda")
    with pytest.raises(hb.HypicError, match="static scratch"):
        hb.seam_advance_noalloc(k, k, k, g, g, seam, R, out, gate=hb.GATE_TOKEN, delta=1, w=8, scale=1.0)
    torch.cuda.synchronize()
    assert bool((R == 3.0).all()) and bool((out == 3.0).all())
