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

import concurrent.futures
import dataclasses
import functools
import math
import os

import numpy as np

GATE_HEAD, GATE_TOKEN, GATE_DIAG = 0, 1, 2



def _e_softplus(sigma: float = 1.0) -> float:
    """E[softplus(sigma Z)] for Z ~ N(0,1), by Gauss-Hermite quadrature."""
    x, w = np.polynomial.hermite_e.hermegauss(80)
    return float(np.sum(w * np.logaddexp(0.0, sigma * x)) / math.sqrt(2.0 * math.pi))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to the nearest bfloat16 (ties to even); result is float32.
    (In 32-bit integer arithmetic: the largest finite pattern plus the rounding bias stays
    below 2^32.)"""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = a.view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    return r.view(np.float32).reshape(a.shape)


_CHUNK = 1 << 21          # values per chunk of a draw


def _draw(ss, shape, post=None):
    """float32 standard normals of `shape`, drawn in chunks of whole leading-axis rows: chunk i
    comes from child i of the SeedSequence `ss` (so the values do not depend on how many
    threads draw them), and `post` (a row-wise map) turns each chunk into the stored float32
    values.  The chunks are drawn and mapped on a thread pool (numpy releases the GIL)."""
    shape = tuple(int(x) for x in shape)
    n = shape[0]
    row = int(np.prod(shape[1:], dtype=np.int64)) if len(shape) > 1 else 1
    per = max(1, _CHUNK // max(row, 1))
    nch = max(1, (n + per - 1) // per)
    kids = ss.spawn(nch)
    out = np.empty(shape, dtype=np.float32)

    def work(i):
        a, b = i * per, min(n, (i + 1) * per)
        if b <= a:
            return
        z = np.random.default_rng(kids[i]).standard_normal((b - a,) + shape[1:], dtype=np.float32)
        out[a:b] = z if post is None else post(z)

    workers = min(16, os.cpu_count() or 1, nch)
    if workers <= 1:
        for i in range(nch):
            work(i)
    else:
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(work, range(nch)))
    return out


def _softplus(x):
    return np.logaddexp(0.0, x)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _unit_rows(x):
    """Rows scaled to unit L2 norm, in float64."""
    x = np.asarray(x, dtype=np.float64)
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


def _tokens(ss_k, ss_v, n_tok, H, dk, dv, *, k_unit, kv_scale, in_dtype):
    """Keys (unit rows, normalised in float64 before rounding, or scaled normals) and values."""
    if k_unit:
        k = _draw(ss_k, (n_tok, H, dk), lambda z: _finish(_unit_rows(z), in_dtype))
    else:
        k = _draw(ss_k, (n_tok, H, dk), lambda z: _finish(z * np.float32(kv_scale), in_dtype))
    vs = np.float32(kv_scale if not k_unit else 1.0)
    v = _draw(ss_v, (n_tok, H, dv), lambda z: _finish(z * vs, in_dtype))
    return k, v


def _unit_q(ss_q, n_tok, H, d, in_dtype):
    return _draw(ss_q, (n_tok, H, d), lambda z: _finish(_unit_rows(z), in_dtype))


def _gdn_tiny(seed, *, stress, n_heads=1, d=16, n_seg=2, seg_len=64, lengths=None):
    """Tiny gated DeltaNet, fp32: 1 head, d=16, 2 segments of 64 tokens."""
    ss_k, ss_v, ss_b, ss_g, ss_q, _ = np.random.SeedSequence(seed).spawn(6)
    lens = np.full(n_seg, seg_len) if lengths is None else np.asarray(lengths)
    N = int(lens.sum())
    k, v = _tokens(ss_k, ss_v, N, n_heads, d, d, k_unit=True, kv_scale=1.0, in_dtype="f32")
    zb = _draw(ss_b, (N, n_heads)).astype(np.float64)
    zg = _draw(ss_g, (N, n_heads)).astype(np.float64)
    if stress:
        beta = _sigmoid(zb - 4.0)
        g = -_softplus(zg) / (float(np.mean(lens)) * _e_softplus())
    else:
        beta = _sigmoid(zb)
        g = -_softplus(zg)
    q = _unit_q(ss_q, N, n_heads, d, "f32")
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
    ss_k, ss_v, ss_q, _ = np.random.SeedSequence(seed).spawn(4)
    lens = np.full(n_seg, seg_len) if lengths is None else np.asarray(lengths)
    N = int(lens.sum())
    k, v = _tokens(ss_k, ss_v, N, n_heads, d, d, k_unit=False, kv_scale=1.0 / math.sqrt(d),
                   in_dtype="bf16")
    g = np.log(retnet_gamma(n_heads)).astype(np.float32)   # decay stays fp32
    qs = np.float32(1.0 / math.sqrt(d))
    q = _draw(ss_q, (N, n_heads, d), lambda z: _finish(z * qs, "bf16"))
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return Workload(name="retnet-8h-d64", n_heads=n_heads, d_k=d, d_v=d, gate=GATE_HEAD,
                    delta=False, in_dtype="bf16", k=k, v=v, g=g, beta=None, seg_start=starts,
                    cache_begin=starts[:-1].copy(), cache_end=starts[1:].copy(), q=q,
                    scale=1.0 / math.sqrt(d),
                    pair_id=np.arange(n_seg, dtype=np.int32)[None, :])


def _gdn_tokens(seed, N, H, d, *, stress, mean_len, gate_scale=0.1):
    ss_k, ss_v, ss_b, ss_g, ss_q, _ = np.random.SeedSequence(seed).spawn(6)
    k, v = _tokens(ss_k, ss_v, N, H, d, d, k_unit=True, kv_scale=1.0, in_dtype="bf16")
    zb = _draw(ss_b, (N, H)).astype(np.float64)
    zg = _draw(ss_g, (N, H)).astype(np.float64)
    if stress:
        beta = _sigmoid(zb - 4.0)
        g = -_softplus(zg) / (mean_len * _e_softplus())
    else:
        beta = _sigmoid(zb)
        g = -_softplus(zg) * gate_scale
    q = _unit_q(ss_q, N, H, d, "bf16")
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
    ss_k, ss_v, ss_b, ss_g, ss_q, ss_p, _ = np.random.SeedSequence(seed).spawn(7)
    rp = np.random.default_rng(ss_p)
    k, v = _tokens(ss_k, ss_v, N, n_heads, d, d, k_unit=True, kv_scale=1.0, in_dtype="bf16")
    zb = _draw(ss_b, (N, n_heads)).astype(np.float64)
    gscale = 1.0 / (float(np.mean(lens)) * _e_softplus(gate_sigma)) if stress else 1.0
    g = _draw(ss_g, (N, n_heads, d),
              lambda z: _finish(-_softplus(z.astype(np.float64) * gate_sigma) * gscale, "bf16"))
    beta = _sigmoid(zb - 4.0) if stress else _sigmoid(zb)
    # the reuse plan has no seam windows, so no token is read out and no q is drawn
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    # chain (request r, layer l) draws n_step ids uniformly from that layer's n_seg pairs;
    # pair index = l * n_seg + segment (one distinct cache copy per layer)
    ids = rp.integers(0, n_seg, size=(n_layers, n_req, n_step)).astype(np.int32)
    ids = ids + (np.arange(n_layers, dtype=np.int32) * n_seg)[:, None, None]
    return Workload(name="kda-32h-d128-131k" + ("-gate-first" if gate_first else "") + ("-stress" if stress else ""),
                    n_heads=n_heads, d_k=d, d_v=d, gate=GATE_DIAG, delta=2 if gate_first else 1,
                    in_dtype="bf16", k=k, v=v,
                    g=g, beta=_finish(beta, "bf16"), seg_start=starts,
                    cache_begin=starts[:-1].copy(), cache_end=starts[1:].copy(), q=None,
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
    if family not in ("gla", "mamba2", "deltanet"):
        raise ValueError(f"unknown family {family!r}")
    ss_k, ss_v, ss_b, ss_g, ss_q, _ = np.random.SeedSequence(seed).spawn(6)
    k, v = _tokens(ss_k, ss_v, N, n_heads, d, d, k_unit=True, kv_scale=1.0, in_dtype=in_dtype)
    mean_len = float(np.mean(lens))
    beta = None
    if family == "gla":
        gate, delta = GATE_DIAG, False
        zg = _draw(ss_g, (N, n_heads, d)).astype(np.float64)
        g = -_softplus(zg) / (mean_len * _e_softplus() if stress else 16.0)
    elif family == "mamba2":
        gate, delta = GATE_TOKEN, False
        zg = _draw(ss_g, (N, n_heads)).astype(np.float64)
        g = -_softplus(zg) / (mean_len * _e_softplus()) if stress else -0.1 * _softplus(zg)
    else:
        gate, delta = GATE_TOKEN, True
        g = np.zeros((N, n_heads))
        zb = _draw(ss_b, (N, n_heads)).astype(np.float64)
        beta = _finish(_sigmoid(zb - 4.0) if stress else _sigmoid(zb), in_dtype)
    q = _unit_q(ss_q, N, n_heads, d, in_dtype)
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
