"""ABI contract on the device: calls are enqueued on the caller's stream and return before
their work runs; a rejected call leaves every buffer as it was."""
import ctypes

import numpy as np
import pytest
import torch

from hybrid_attention_prefill_amd import binding as hb
from hybrid_attention_prefill_amd import workloads as wl
from _util import dev, workload_tensors

pytestmark = pytest.mark.gpu


def _busy(n=6):
    """About 100 ms of fp32 products on the current stream."""
    a = torch.full((8192, 8192), 1e-4, device="cuda")
    c = torch.empty_like(a)
    for _ in range(n):
        torch.mm(a, a, out=c)
    return c


def test_calls_are_asynchronous_on_the_given_stream():
    """On a side stream: products that keep it busy, then the copy that fills v, then the
    build and the composition.  The library calls return while that stream still has work
    queued, and their results are those of the same calls on the default stream with v
    already in place -- so they ran on the side stream, after the copy."""
    W = wl.make("gdn-16h-d128-32k", stress=True, n_heads=2, lengths=[700, 300])
    x = workload_tensors(W)
    sb, se = dev(W.cache_begin, torch.int64), dev(W.cache_end, torch.int64)
    ids = dev(W.pair_id, torch.int32)
    T_ref, S_ref = hb.segment_build(x["k"], x["v"], x["g"], x["beta"], sb, se, gate=W.gate, delta=W.delta,
                                    t_layout=hb.T_SPLIT)
    R_ref = torch.zeros((1, 2, 128, 128), device="cuda")
    hb.compose(T_ref, S_ref, ids, R_ref)
    v_late = torch.zeros_like(x["v"])
    T = torch.empty_like(T_ref)
    S = torch.empty_like(S_ref)
    R = torch.zeros_like(R_ref)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        _busy()
        v_late.copy_(x["v"])
    hb.segment_build(x["k"], v_late, x["g"], x["beta"], sb, se, gate=W.gate, delta=W.delta,
                     t_layout=hb.T_SPLIT, T_out=T, S_out=S, stream=s)
    hb.compose(T, S, ids, R, stream=s)
    pending = not s.query()
    s.synchronize()
    assert pending, "the side stream had finished before the calls returned"
    assert torch.equal(T, T_ref) and torch.equal(S, S_ref) and torch.equal(R, R_ref)


def test_rejected_calls_leave_buffers_untouched():
    """Argument errors are reported before anything is launched: outputs keep their
    contents (checked after a device synchronisation)."""
    lib = hb.load_library()
    W = wl.make("gdn-16h-d128-32k", n_heads=2, lengths=[1500, 200])   # long enough to use a workspace
    assert hb.build_workspace_bytes(2, 128, 128, 2, W.n_tokens) > 1
    x = workload_tensors(W)
    sb, se = dev(W.cache_begin, torch.int64), dev(W.cache_end, torch.int64)
    T = torch.full((2, 2, 128, 128), 7.0, device="cuda")
    S = torch.full((2, 2, 128, 128), 7.0, device="cuda")
    ws = torch.zeros(256, device="cuda", dtype=torch.uint8)   # far too small
    d = hb.make_dims(2, 128, 128, gate=hb.GATE_TOKEN, delta=1, in_dtype=hb.BF16)
    st = lib.hypic_segment_build(ctypes.byref(d), 2, hb._ptr(sb), hb._ptr(se), W.n_tokens, hb._ptr(x["k"]),
                                 hb._ptr(x["v"]), hb._ptr(x["g"]), hb._ptr(x["beta"]), hb._ptr(T), hb._ptr(S),
                                 hb._ptr(ws), 1, None)
    assert st == hb.HYPIC_E_INVALID
    bad = hb.make_dims(2, 128, 128, gate=hb.GATE_TOKEN, delta=7, in_dtype=hb.BF16)
    st = lib.hypic_segment_build(ctypes.byref(bad), 2, hb._ptr(sb), hb._ptr(se), W.n_tokens, hb._ptr(x["k"]),
                                 hb._ptr(x["v"]), hb._ptr(x["g"]), hb._ptr(x["beta"]), hb._ptr(T), hb._ptr(S),
                                 None, 0, None)
    assert st == hb.HYPIC_E_INVALID
    R = torch.full((1, 2, 128, 128), 3.0, device="cuda")
    ids = dev(np.array([[0, 1]], np.int32), torch.int32)
    st = lib.hypic_compose(ctypes.byref(bad), 1, 2, hb._ptr(ids), 2, hb._ptr(T), hb._ptr(S), hb._ptr(R), None)
    assert st == hb.HYPIC_E_INVALID
    st = lib.hypic_compose(ctypes.byref(d), 1, 2, None, 2, hb._ptr(T), hb._ptr(S), hb._ptr(R), None)
    assert st == hb.HYPIC_E_INVALID
    torch.cuda.synchronize()
    assert bool((T == 7.0).all()) and bool((S == 7.0).all()) and bool((R == 3.0).all())
