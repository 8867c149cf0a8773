"""Seeded synthetic workloads for the segment build / compose / seam path.

This module holds the input recipe only -- random draws, normalisation of the
drawn keys, the gate and beta transforms of the drawn numbers, rounding to the
input dtype, segment lengths and reuse plans.  It contains none of the state
arithmetic of the method, and it is the only module shared by the GPU tests and
the CPU oracle's tests.

The workloads follow the shapes the pages give for HYPIC's prompts (tens
to hundreds of independent segments, segments usually longer than 512 tokens,
32k and 100k-token prompts, 30 linear layers in a hybrid model) with the value
distributions listed below.  They stand in for the public datasets and the
production trace the pages evaluate on, none of which is used here.

Every array is float32 holding values exactly representable in the input dtype
(bf16 values are rounded to nearest-even from fp32), so the GPU path and the
oracle consume bit-identical inputs.
"""
from __future__ import annotations

import dataclasses
import functools
import math

import numpy as np

GATE_HEAD, GATE_TOKEN, GATE_DIAG = 0, 1, 2



def _e_softplus(sigma: float = 1.0) -> float:
    """E[softplus(sigma Z)] for Z ~ N(0,1), by Gauss-Hermite quadrature."""
    x, w = np.polynomial.hermite_e.hermegauss(80)
    return float(np.sum(w * np.logaddexp(0.0, sigma * x)) / math.sqrt(2.0 * math.pi))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); result is float32."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def _softplus(x):
    return np.logaddexp(0.0, x)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


@dataclasses.dataclass
class Workload:
    """Inputs and plan for one synthetic workload.

    Token arrays are packed over the whole prompt: q, k [N, H, d_k], v [N, H, d_v],
    beta [N, H]; g is [H] (head-constant decay), [N, H] (token scalar gate) or
    [N, H, d_k] (token per-channel gate).  Gates are log-gates (<= 0).
    Segment i spans tokens [seg_start[i], seg_start[i+1]); its cached part is
    [cache_begin[i], cache_end[i]) (all of it, or all but the seam window).
    """
    name: str
    n_heads: int
    d_k: int
    d_v: int
    gate: int
    delta: int                    # 0 plain write, 1 erase then gate, 2 gate then erase
    in_dtype: str                 # "f32" or "bf16"
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray | None
    seg_start: np.ndarray         # int64 [n_seg + 1]
    cache_begin: np.ndarray       # int64 [n_seg]
    cache_end: np.ndarray         # int64 [n_seg]
    q: np.ndarray | None = None
    scale: float = 1.0
    w: int = 0                    # seam window length (0: no seams)
    seam_start: np.ndarray | None = None   # int64 [n_chain, n_step], -1 = none
    pair_id: np.ndarray | None = None      # int32 [n_chain, n_step], -1 = skip
    cold: np.ndarray | None = None         # bool [n_seg]
    n_layers: int = 1
    notes: str = ""

    @property
    def n_tokens(self) -> int:
        return int(self.k.shape[0])

    @property
    def n_seg(self) -> int:
        return int(self.cache_begin.shape[0])

    @property
    def seg_len(self) -> np.ndarray:
        return np.diff(self.seg_start)


def _finish(x, in_dtype):
    x = np.asarray(x, dtype=np.float32)
    return round_bf16(x) if in_dtype == "bf16" else x


def _tokens(rng_k, rng_v, n_tok, H, dk, dv, *, k_unit, kv_scale, in_dtype):
    k = rng_k.standard_normal((n_tok, H, dk))
    k = _unit_rows(k) if k_unit else k * kv_scale
    v = rng_v.standard_normal((n_tok, H, dv)) * (kv_scale if not k_unit else 1.0)
    return _finish(k, in_dtype), _finish(v, in_dtype)


def _gdn_tiny(seed, *, stress, n_heads=1, d=16, n_seg=2, seg_len=64, lengths=None):
    """Tiny gated DeltaNet, fp32: 1 head, d=16, 2 segments of 64 tokens."""
    ss = np.random.SeedSequence(seed).spawn(6)
    rk, rv, rb, rg, rq, _ = [np.random.default_rng(s) for s in ss]
    lens = np.full(n_seg, seg_len) if lengths is None else np.asarray(lengths)
    N = int(lens.sum())
    k, v = _tokens(rk, rv, N, n_heads, d, d, k_unit=True, kv_scale=1.0, in_dtype="f32")
    zb = rb.standard_normal((N, n_heads))
    zg = rg.standard_normal((N, n_heads))
    if stress:
        beta = _sigmoid(zb - 4.0)
        g = -_softplus(zg) / (float(np.mean(lens)) * _e_softplus())
    else:
        beta = _sigmoid(zb)
        g = -_softplus(zg)
    q = _finish(_unit_rows(rq.standard_normal((N, n_heads, d))), "f32")
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return Workload(name="gdn-tiny-f32" + ("-stress" if stress else ""), n_heads=n_heads,
                    d_k=d, d_v=d, gate=GATE_TOKEN, delta=True, in_dtype="f32", k=k, v=v,
                    g=_finish(g, "f32"), beta=_finish(beta, "f32"), seg_start=starts,
                    cache_begin=starts[:-1].copy(), cache_end=starts[1:].copy(), q=q,
                    scale=1.0 / math.sqrt(d),
                    pair_id=np.arange(n_seg, dtype=np.int32)[None, :])


def retnet_gamma(n_heads):
    """gamma_h = 1 - 2^(-5-h)."""
    return 1.0 - 2.0 ** (-5.0 - np.arange(n_heads, dtype=np.float64))


def _retnet(seed, *, stress, n_heads=8, d=64, n_seg=16, seg_len=512, lengths=None):
    """RetNet-style scalar decay, bf16 k/v, fp32 decay: 8 heads, d=64, 16 x 512."""
    ss = np.random.SeedSequence(seed).spawn(4)
    rk, rv, rq, _ = [np.random.default_rng(s) for s in ss]
    lens = np.full(n_seg, seg_len) if lengths is None else np.asarray(lengths)
    N = int(lens.sum())
    k, v = _tokens(rk, rv, N, n_heads, d, d, k_unit=False, kv_scale=1.0 / math.sqrt(d),
                   in_dtype="bf16")
    g = np.log(retnet_gamma(n_heads)).astype(np.float32)   # decay stays fp32
    q = _finish(rq.standard_normal((N, n_heads, d)) / math.sqrt(d), "bf16")
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return Workload(name="retnet-8h-d64", n_heads=n_heads, d_k=d, d_v=d, gate=GATE_HEAD,
                    delta=False, in_dtype="bf16", k=k, v=v, g=g, beta=None, seg_start=starts,
                    cache_begin=starts[:-1].copy(), cache_end=starts[1:].copy(), q=q,
                    scale=1.0 / math.sqrt(d),
                    pair_id=np.arange(n_seg, dtype=np.int32)[None, :])


def _gdn_tokens(seed, N, H, d, *, stress, mean_len, gate_scale=0.1):
    ss = np.random.SeedSequence(seed).spawn(6)
    rk, rv, rb, rg, rq, _ = [np.random.default_rng(s) for s in ss]
    k, v = _tokens(rk, rv, N, H, d, d, k_unit=True, kv_scale=1.0, in_dtype="bf16")
    zb = rb.standard_normal((N, H))
    zg = rg.standard_normal((N, H))
    if stress:
        beta = _sigmoid(zb - 4.0)
        g = -_softplus(zg) / (mean_len * _e_softplus())
    else:
        beta = _sigmoid(zb)
        g = -_softplus(zg) * gate_scale
    q = _finish(_unit_rows(rq.standard_normal((N, H, d))), "bf16")
    return k, v, _finish(beta, "bf16"), _finish(g, "bf16"), q


def _gdn_32k(seed, *, stress, n_heads=16, d=128, n_seg=32, seg_len=1024, lengths=None):
    """Gated DeltaNet, bf16 inputs: 16 heads, d=128, 32 segments x 1024 tokens."""
    lens = np.full(n_seg, seg_len) if lengths is None else np.asarray(lengths)
    N = int(lens.sum())
    k, v, beta, g, q = _gdn_tokens(seed, N, n_heads, d, stress=stress, mean_len=float(np.mean(lens)))
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return Workload(name="gdn-16h-d128-32k" + ("-stress" if stress else ""), n_heads=n_heads, d_k=d,
                    d_v=d, gate=GATE_TOKEN, delta=True, in_dtype="bf16", k=k, v=v, g=g, beta=beta,
                    seg_start=starts, cache_begin=starts[:-1].copy(), cache_end=starts[1:].copy(),
                    q=q, scale=1.0 / math.sqrt(d),
                    pair_id=np.arange(len(lens), dtype=np.int32)[None, :])


def lognormal_lengths(seed, n_seg=128, total=100_000, median=700, sigma=0.5, minimum=512):
    """Segment lengths max(minimum, floor(median * exp(sigma z))), then adjusted one
    token at a time, round-robin, until they sum to `total` (removals only from
    segments longer than `minimum`)."""
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(8)[7])
    z = rng.standard_normal(n_seg)
    L = np.maximum(minimum, np.floor(median * np.exp(sigma * z))).astype(np.int64)
    i = 0
    guard = 0
    while L.sum() != total:
        if L.sum() < total:
            L[i % n_seg] += 1
        elif L[i % n_seg] > minimum:
            L[i % n_seg] -= 1
        i += 1
        guard += 1
        if guard > 100 * total:
            raise ValueError("cannot reach the requested total")
    return L


def _gdn_100k_seam(seed, *, stress, n_heads=16, d=128, n_seg=128, total=100_000, w=8, minimum=512,
          median=700, cold_frac=0.2):
    """Gated DeltaNet 100k-token prompt: 128 lognormal segments (median 700, min 512),
    80% warm / 20% cold, seam window w=8 at every internal segment."""
    lens = lognormal_lengths(seed, n_seg=n_seg, total=total, median=median, minimum=minimum)
    N = int(lens.sum())
    k, v, beta, g, q = _gdn_tokens(seed, N, n_heads, d, stress=stress, mean_len=float(np.mean(lens)))
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    cb = starts[:-1].copy()
    cb[1:] += w                     # internal segments: the seam window is not cached
    ce = starts[1:].copy()
    seam = starts[:-1].copy()[None, :].astype(np.int64)
    seam[0, 0] = -1                 # the first segment has no seam
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(9)[8])
    n_cold = int(round(cold_frac * n_seg))
    cold = np.zeros(n_seg, dtype=bool)
    cold[rng.permutation(n_seg)[:n_cold]] = True
    return Workload(name="gdn-16h-d128-100k-seam" + ("-stress" if stress else ""), n_heads=n_heads,
                    d_k=d, d_v=d, gate=GATE_TOKEN, delta=True, in_dtype="bf16", k=k, v=v, g=g,
                    beta=beta, seg_start=starts, cache_begin=cb, cache_end=ce, q=q,
                    scale=1.0 / math.sqrt(d), w=w, seam_start=seam,
                    pair_id=np.arange(n_seg, dtype=np.int32)[None, :], cold=cold)


def _kda_131k(seed, *, stress, n_heads=32, d=128, n_seg=64, seg_len=2048, n_req=64, n_step=256,
          n_layers=30, lengths=None, gate_first=False, gate_sigma=0.05):
    """KDA-style per-channel gate, bf16: 32 heads, d=128, 64 x 2048 tokens; then
    n_req requests x n_step cached segments per layer x n_layers layers.
    gate_first: the gate applied before the erase (delta 2) instead of after it;
    gate_sigma: spread of the per-channel log-gates, g = -softplus(gate_sigma z)."""
    lens = np.full(n_seg, seg_len) if lengths is None else np.asarray(lengths)
    N = int(lens.sum())
    ss = np.random.SeedSequence(seed).spawn(7)
    rk, rv, rb, rg, rq, rp, _ = [np.random.default_rng(s) for s in ss]
    k, v = _tokens(rk, rv, N, n_heads, d, d, k_unit=True, kv_scale=1.0, in_dtype="bf16")
    zb = rb.standard_normal((N, n_heads))
    zg = rg.standard_normal((N, n_heads, d))
    if stress:
        beta = _sigmoid(zb - 4.0)
        g = -_softplus(zg * gate_sigma) / (float(np.mean(lens)) * _e_softplus(gate_sigma))
    else:
        beta = _sigmoid(zb)
        g = -_softplus(zg * gate_sigma)
    q = _finish(_unit_rows(rq.standard_normal((N, n_heads, d))), "bf16")
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    # chain (request r, layer l) draws n_step ids uniformly from that layer's n_seg pairs;
    # pair index = l * n_seg + segment (one distinct cache copy per layer)
    ids = rp.integers(0, n_seg, size=(n_layers, n_req, n_step)).astype(np.int32)
    ids = ids + (np.arange(n_layers, dtype=np.int32) * n_seg)[:, None, None]
    return Workload(name="kda-32h-d128-131k" + ("-gate-first" if gate_first else "") + ("-stress" if stress else ""),
                    n_heads=n_heads, d_k=d, d_v=d, gate=GATE_DIAG, delta=2 if gate_first else 1,
                    in_dtype="bf16", k=k, v=v,
                    g=_finish(g, "bf16"), beta=_finish(beta, "bf16"), seg_start=starts,
                    cache_begin=starts[:-1].copy(), cache_end=starts[1:].copy(), q=q,
                    scale=1.0 / math.sqrt(d), pair_id=ids.reshape(n_layers * n_req, n_step),
                    n_layers=n_layers)


def _variant(family, seed, *, stress, n_heads=16, d=None, n_seg=16, seg_len=1024, lengths=None,
             in_dtype="bf16"):
    """The other transition families, 16 segments x 1024 tokens of bf16 inputs:
      gla      : per-channel gate, no erase; g = -softplus(z) / 16 (log-sigmoid gates
                 with temperature 16), d = 128;
      mamba2   : token scalar gate, no erase; g = -0.1 softplus(z), d = 64;
      deltanet : erase and write with beta = sigmoid(z), no gate (g = 0), d = 128.
    Stress: gates scaled to a mean total log-decay of -1 per segment, beta = sigmoid(z - 4)."""
    d = (64 if family == "mamba2" else 128) if d is None else d
    lens = np.full(n_seg, seg_len) if lengths is None else np.asarray(lengths)
    N = int(lens.sum())
    ss = np.random.SeedSequence(seed).spawn(6)
    rk, rv, rb, rg, rq, _ = [np.random.default_rng(s) for s in ss]
    k, v = _tokens(rk, rv, N, n_heads, d, d, k_unit=True, kv_scale=1.0, in_dtype=in_dtype)
    mean_len = float(np.mean(lens))
    beta = None
    if family == "gla":
        gate, delta = GATE_DIAG, False
        zg = rg.standard_normal((N, n_heads, d))
        g = -_softplus(zg) / (mean_len * _e_softplus() if stress else 16.0)
    elif family == "mamba2":
        gate, delta = GATE_TOKEN, False
        zg = rg.standard_normal((N, n_heads))
        g = -_softplus(zg) / (mean_len * _e_softplus()) if stress else -0.1 * _softplus(zg)
    elif family == "deltanet":
        gate, delta = GATE_TOKEN, True
        g = np.zeros((N, n_heads))
        zb = rb.standard_normal((N, n_heads))
        beta = _finish(_sigmoid(zb - 4.0) if stress else _sigmoid(zb), in_dtype)
    else:
        raise ValueError(f"unknown family {family!r}")
    q = _finish(_unit_rows(rq.standard_normal((N, n_heads, d))), in_dtype)
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    name = {"gla": "gla-16h-d128-16k", "mamba2": "mamba2-16h-d64-16k",
            "deltanet": "deltanet-16h-d128-16k"}[family]
    return Workload(name=name + ("-stress" if stress else ""), n_heads=n_heads, d_k=d, d_v=d,
                    gate=gate, delta=delta, in_dtype=in_dtype, k=k, v=v, g=_finish(g, in_dtype),
                    beta=beta, seg_start=starts, cache_begin=starts[:-1].copy(),
                    cache_end=starts[1:].copy(), q=q, scale=1.0 / math.sqrt(d),
                    pair_id=np.arange(len(lens), dtype=np.int32)[None, :])


# name -> (maker, default seed)
_MAKERS = {
    "gdn-tiny-f32": (_gdn_tiny, 1),
    "retnet-8h-d64": (_retnet, 2),
    "gdn-16h-d128-32k": (_gdn_32k, 3),
    "gdn-16h-d128-100k-seam": (_gdn_100k_seam, 4),
    "kda-32h-d128-131k": (_kda_131k, 5),
    "gla-16h-d128-16k": (functools.partial(_variant, "gla"), 6),
    "mamba2-16h-d64-16k": (functools.partial(_variant, "mamba2"), 7),
    "deltanet-16h-d128-16k": (functools.partial(_variant, "deltanet"), 8),
}
NAMES = tuple(_MAKERS)


def make(name: str, *, stress: bool = False, seed: int | None = None, **overrides) -> Workload:
    """Build the named workload (see NAMES).  Keyword overrides shrink a workload for
    tests (n_heads, n_seg, seg_len, lengths, total, n_req, n_step, n_layers, ...)."""
    if name not in _MAKERS:
        raise ValueError(f"unknown workload {name!r}; one of {', '.join(_MAKERS)}")
    maker, default_seed = _MAKERS[name]
    return maker(default_seed if seed is None else seed, stress=stress, **overrides)
