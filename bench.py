#!/usr/bin/env python3
"""Benchmark of the HYPIC linear-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step = one pass of the hot path over one synthetic request with all inputs
resident in HBM:

* gdn-16h-d128-100k-seam (default): a 100,000-token prompt of 128 lognormal
  segments (16 gated-DeltaNet heads, d = 128, bf16): build (T_C, S(C|0)) for
  the 26 cold segments, then one seam-advance call that steps the w = 8 seam
  window of every internal segment (emitting its outputs) and composes all 128
  cached pairs in order.  Warm pairs come from an untimed earlier build.
* retnet-8h-d64, gdn-16h-d128-32k, kda-32h-d128-131k: build every segment,
  then compose as the workload says (kda-32h-d128-131k: 64 requests x 256
  cached segments per layer x 30 layers).

Prints one JSON line.  `value` is segment-build tokens/s (tokens built per
second of build-kernel time); `compose_us_per_segment` is the chain kernel time
per (request, segment, layer) with all heads; `roofline` is for the kernel
with the largest share of the step, from HIP events on the stream the library
launches on.  `cpu_baseline` times the fp64 oracle (test infrastructure) on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 / fp16 MFMA
METRIC = "segment-build tokens/s + compose µs/segment on 1 GPU, % of MFMA/HBM roofline"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="gdn-16h-d128-100k-seam",
                   choices=["retnet-8h-d64", "gdn-16h-d128-32k", "gdn-16h-d128-100k-seam", "kda-32h-d128-131k"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="before warm-up, copy MIB MiB device-to-device once (a plain copy kernel of known "
                        "size, the reference for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


class Timer:
    """HIP-event timing of library calls on the current stream.

    The events are created with hipEventDisableSystemFence: timing-only events.  A default
    event's record ends with a system-scope fence (cache write-back and invalidation), which
    costs the GPU about 5 us per record and lands inside the measured interval; the elapsed
    times are read only after a device synchronisation, which is all these events need."""

    DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence

    def __init__(self, torch):
        self.torch = torch
        self.pending = {}
        self.totals = {}
        self.counts = {}
        # the HIP runtime torch and the library already share (same soname)
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.free = []

    def _event(self):
        if self.free:
            return self.free.pop()
        ev = ctypes.c_void_p()
        if self.hip.hipEventCreateWithFlags(ctypes.byref(ev), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return ev

    def run(self, name, fn):
        stream = ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream)
        s, e = self._event(), self._event()
        if self.hip.hipEventRecord(s, stream) != 0:
            raise RuntimeError("hipEventRecord failed")
        fn()
        if self.hip.hipEventRecord(e, stream) != 0:
            raise RuntimeError("hipEventRecord failed")
        self.pending.setdefault(name, []).append((s, e))

    def collect(self):
        self.torch.cuda.synchronize()
        ms = ctypes.c_float()
        for name, evs in self.pending.items():
            for s, e in evs:
                if self.hip.hipEventElapsedTime(ctypes.byref(ms), s, e) != 0:
                    raise RuntimeError("hipEventElapsedTime failed")
                self.totals[name] = self.totals.get(name, 0.0) + ms.value * 1e-3
                self.counts[name] = self.counts.get(name, 0) + 1
                self.free += [s, e]
        self.pending = {}

    def reset(self):
        for evs in self.pending.values():
            for s, e in evs:
                self.free += [s, e]
        self.pending, self.totals, self.counts = {}, {}, {}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU path is not part "
              "of this build.", file=sys.stderr)
        return 1
    import torch

    from hybrid_attention_prefill_amd import binding as hb
    from hybrid_attention_prefill_amd import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    W = wl.make(args.workload)
    seam_plan = W.seam_start is not None
    layered = W.n_layers > 1
    H, d = W.n_heads, W.d_k
    dt = torch.bfloat16 if W.in_dtype == "bf16" else torch.float32
    T = lambda a, t: torch.from_numpy(np.ascontiguousarray(a)).to(device=dev, dtype=t)
    k, v = T(W.k, dt), T(W.v, dt)
    g = T(W.g, torch.float32 if W.gate == 0 else dt)
    beta = T(W.beta, dt) if W.beta is not None else None
    q = T(W.q, dt) if W.q is not None else None
    in_bytes = 2 if W.in_dtype == "bf16" else 4
    gate_elems = {0: 0, 1: 1, 2: d}[W.gate]
    # constant decay caches T as one number; dense T is cached in the composition kernels'
    # operand format (bf16 hi/lo planes, 4 bytes per entry like fp32)
    t_layout = hb.T_SCALAR if W.gate == hb.GATE_HEAD else hb.T_SPLIT
    tsz = 1 if t_layout == hb.T_SCALAR else d * d
    tdt = torch.bfloat16 if t_layout == hb.T_SPLIT else torch.float32
    tshape = lambda n: (n, H) if t_layout == hb.T_SCALAR else (n, H, 2, d * d)

    def build_workspace(n_seg):   # allocated outside the timed region (None: no cutting)
        nb = hb.build_workspace_bytes(H, d, d, n_seg, W.n_tokens, gate=W.gate, delta=W.delta,
                                      in_dtype=hb.BF16 if W.in_dtype == "bf16" else hb.F32)
        return torch.empty(nb, device=dev, dtype=torch.uint8) if nb > 0 else None
    timer = Timer(torch)
    info = {}

    if seam_plan:
        cold = np.flatnonzero(W.cold)
        warm = np.flatnonzero(~W.cold)
        order = np.concatenate([warm, cold])           # cache slots: warm pairs first, cold last
        slot = np.empty(W.n_seg, dtype=np.int32)
        slot[order] = np.arange(W.n_seg, dtype=np.int32)
        Tc = torch.empty(tshape(W.n_seg), device=dev, dtype=tdt)
        Sc = torch.empty((W.n_seg, H, d, d), device=dev)
        sb_all, se_all = T(W.cache_begin[order], torch.int64), T(W.cache_end[order], torch.int64)
        hb.segment_build(k, v, g, beta, sb_all, se_all, gate=W.gate, delta=W.delta, t_layout=t_layout,
                         T_out=Tc, S_out=Sc)
        n_warm = len(warm)
        sb_c, se_c = T(W.cache_begin[cold], torch.int64), T(W.cache_end[cold], torch.int64)
        Tcold, Scold = Tc[n_warm:], Sc[n_warm:]
        ids = T(slot[None, :], torch.int32)
        seam = T(W.seam_start, torch.int64)
        R = torch.zeros((1, H, d, d), device=dev)
        out = torch.zeros((1, W.n_seg, W.w, H, d), device=dev)
        ws = torch.empty(hb.seam_workspace_bytes(H, d, d, 1, W.n_seg, W.w), device=dev, dtype=torch.uint8)
        wsb = build_workspace(len(cold))
        cold_tokens = int((W.cache_end[cold] - W.cache_begin[cold]).sum())

        def step():
            timer.run("segment_build", lambda: hb.segment_build(k, v, g, beta, sb_c, se_c, gate=W.gate,
                                                                delta=W.delta, t_layout=t_layout,
                                                                T_out=Tcold, S_out=Scold, workspace=wsb))
            R.zero_()
            timer.run("seam_advance", lambda: hb.seam_advance(q, k, v, g, beta, seam, R, out, gate=W.gate,
                                                              delta=W.delta, w=W.w, scale=W.scale, pair_id=ids,
                                                              T_cache=Tc, S_cache=Sc, workspace=ws))

        built_tokens = cold_tokens
        prefill_segs = (sb_c, se_c)
        n_segments_composed = W.n_seg
        n_windows = int((W.seam_start >= 0).sum())
        work = {
            "segment_build": dict(
                bytes=cold_tokens * H * (2 * d * in_bytes + 2 * in_bytes) + len(cold) * H * (d * d + d * d) * 4,
                flops=cold_tokens * H * 4 * d * (d + d)),
            "seam_advance": dict(
                bytes=W.n_seg * H * (d * d + d * d) * 4 + n_windows * W.w * H * ((3 * d + 2) * in_bytes + d * 4),
                flops=W.n_seg * H * 2 * d * d * d + n_windows * W.w * H * 6 * d * d),
        }
        info.update(cold_segments=int(len(cold)), cold_tokens=cold_tokens, seam_windows=n_windows, w=W.w)
    else:
        sb, se = T(W.cache_begin, torch.int64), T(W.cache_end, torch.int64)
        Tb = torch.empty(tshape(W.n_seg), device=dev, dtype=tdt)
        Sb = torch.empty((W.n_seg, H, d, d), device=dev)
        if layered:
            # one distinct cache copy per layer, so re-reads are not served from the 256 MB MALL
            Tc = torch.empty(tshape(W.n_layers * W.n_seg), device=dev, dtype=tdt)
            Sc = torch.empty((W.n_layers * W.n_seg, H, d, d), device=dev)
        else:
            Tc, Sc = Tb, Sb
        ids = T(W.pair_id, torch.int32)
        n_chain, n_step = W.pair_id.shape
        R = torch.zeros((n_chain, H, d, d), device=dev)
        built_tokens = int((W.cache_end - W.cache_begin).sum())
        prefill_segs = (sb, se)

        if layered:
            # the 30 per-layer caches: copies of one untimed earlier build
            hb.segment_build(k, v, g, beta, sb, se, gate=W.gate, delta=W.delta, t_layout=t_layout,
                             T_out=Tb, S_out=Sb)
            for l in range(W.n_layers):
                Tc[l * W.n_seg:(l + 1) * W.n_seg].copy_(Tb)
                Sc[l * W.n_seg:(l + 1) * W.n_seg].copy_(Sb)

        wsb = build_workspace(W.n_seg)

        def step():
            timer.run("segment_build", lambda: hb.segment_build(k, v, g, beta, sb, se, gate=W.gate, delta=W.delta,
                                                                t_layout=t_layout, T_out=Tb, S_out=Sb,
                                                                workspace=wsb))
            R.zero_()
            timer.run("compose", lambda: hb.compose(Tc, Sc, ids, R, t_layout=t_layout))

        n_segments_composed = n_chain * n_step
        work = {
            "segment_build": dict(
                bytes=built_tokens * H * (2 * d * in_bytes + (gate_elems + 1) * in_bytes)
                + W.n_seg * H * (tsz + d * d) * 4,
                flops=built_tokens * H * (2 * d * d if W.gate == hb.GATE_HEAD else 4 * d * (d + d))),
            "compose": dict(bytes=n_segments_composed * H * (tsz + d * d) * 4,
                            flops=n_segments_composed * H * (2 * d * d if tsz == 1 else 2 * d * d * d)),
        }
        info.update(segments=W.n_seg, built_tokens=built_tokens, chains=n_chain, steps_per_chain=n_step,
                    layers=W.n_layers)

    if args.calibrate_copy > 0:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timer.reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timer.collect()

    # After the timed steps: the fused cold prefill of the same (built) segments, with and
    # without T -- T's share of the linear layer's prefill on these segments (outputs need
    # each token's prefix state, so these segments are not cut).
    prefill = None
    if W.gate == hb.GATE_TOKEN and W.delta and W.in_dtype == "bf16" and d in (64, 128):
        pb, pe = prefill_segs
        n_pf = pb.shape[0]
        pout = torch.empty((W.n_tokens, H, d), device=dev)
        pS = torch.empty((n_pf, H, d, d), device=dev)
        pT = torch.empty(tshape(n_pf), device=dev, dtype=tdt)
        calls = {
            "with_T": lambda: hb.segment_prefill(q, k, v, g, beta, pb, pe, scale=W.scale, t_layout=t_layout,
                                                 T_out=pT, S_out=pS, out=pout),
            "S_only": lambda: hb.segment_prefill(q, k, v, g, beta, pb, pe, scale=W.scale, want_T=False,
                                                 S_out=pS, out=pout),
        }
        ptimer = Timer(torch)
        for _ in range(2):
            for fn in calls.values():
                fn()
        torch.cuda.synchronize()
        for _ in range(max(3, min(args.steps, 10))):
            for name, fn in calls.items():
                ptimer.run(name, fn)
        ptimer.collect()
        pt = {name: ptimer.totals[name] / ptimer.counts[name] for name in calls}
        prefill = {"with_T_us": round(pt["with_T"] * 1e6, 2), "S_only_us": round(pt["S_only"] * 1e6, 2),
                   "T_overhead": round(pt["with_T"] / pt["S_only"] - 1, 4),
                   "tokens_per_s_with_T": round(built_tokens / pt["with_T"], 1)}

    kern = {}
    for name, tot in timer.totals.items():
        avg = tot / timer.counts[name]
        wk = work[name]
        gbs = wk["bytes"] / avg / 1e9
        tfs = wk["flops"] / avg / 1e12
        kern[name] = dict(avg_us=round(avg * 1e6, 2), alg_bytes=int(wk["bytes"]), alg_flops=int(wk["flops"]),
                          GBps=round(gbs, 1), TFLOPps=round(tfs, 2), hbm_frac=round(gbs / HBM_PEAK_GBS, 4),
                          mfma_frac=round(tfs / MFMA_BF16_PEAK_TFLOPS, 4))
    build_avg = timer.totals["segment_build"] / timer.counts["segment_build"]
    chain_name = "seam_advance" if "seam_advance" in kern else "compose"
    chain_avg = timer.totals[chain_name] / timer.counts[chain_name]
    dom = max(kern, key=lambda n: kern[n]["avg_us"])
    dk = kern[dom]
    roofline = {"bound": "hbm", "achieved": dk["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dk["GBps"] / HBM_PEAK_GBS, 4), "traffic": measured_traffic(W.name, dom),
                "kernel": dom}

    line = {
        "metric": METRIC,
        "value": round(built_tokens / build_avg, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": W.in_dtype,
        "data": "synthetic",
        "config": {"workload": W.name, "heads": H, "d_k": d, "d_v": d,
                   "t_cache": {hb.T_SCALAR: "scalar f32", hb.T_SPLIT: "bf16 hi/lo planes"}[t_layout], **info},
        "compose_us_per_segment": round(chain_avg / (n_segments_composed) * 1e6, 4),
        "build_us": round(build_avg * 1e6, 2),
        "kernels": kern,
        "roofline": roofline,
    }
    if prefill is not None:
        line["prefill"] = prefill
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(W)
    print(json.dumps(line), flush=True)
    return 0


# Sources of the kernels each library call launches (a stored counter measurement is
# reported only while these files are unchanged).
CALL_SOURCES = {
    "seam_advance": ["seam.hip", "seam_chain.hip", "seam_layout.h", "compose.hip", "hypic_device.h", "hypic_kernels.h"],
    "compose": ["compose.hip", "hypic_device.h", "hypic_kernels.h"],
    "segment_build": ["build_gdn.hip", "build_split.hip", "build_kda.hip", "build_decay.hip", "build_common.h",
                      "hypic_device.h", "hypic_kernels.h"],
}


def sources_digest(call):
    import hashlib
    h = hashlib.sha256()
    for f in CALL_SOURCES[call]:
        with open(os.path.join(ROOT, "hybrid_attention_prefill_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, call):
    """HBM bytes per call from the stored rocprofv3 FETCH_SIZE + WRITE_SIZE passes
    (profiles/traffic_<workload>.md), or None when there is none for this call or the
    kernels' sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        for ln in fh:
            if ln.startswith("traffic-json: "):
                rec = json.loads(ln[len("traffic-json: "):])
                if rec.get("call") == call and rec.get("sources") == sources_digest(call):
                    return int(rec["bytes_per_call"])
    return None


def cpu_baseline(W):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload:
    a few of the segments the step builds, all heads (8 of them for the 32-head
    workload), packed and converted to fp64 before the clock starts."""
    import oracle
    n_thr = oracle.num_threads()
    # about 10 s on 8-16 cores: the 100k prompt builds every segment (as for a fully cold
    # request), the 32k workload 24 of its 32 segments, the others a handful
    pool = np.arange(W.n_seg)
    segs = {"retnet-8h-d64": pool, "gdn-16h-d128-32k": pool[:24], "gdn-16h-d128-100k-seam": pool,
            "kda-32h-d128-131k": pool[:6]}[W.name]
    heads = W.n_heads if W.n_heads <= 16 else 8
    parts = [np.arange(W.cache_begin[s], W.cache_end[s]) for s in segs]
    idx = np.concatenate(parts)
    lens = np.array([len(p) for p in parts])
    ends = np.cumsum(lens)
    f64 = lambda a: np.ascontiguousarray(a, dtype=np.float64)
    k, v = f64(W.k[idx, :heads]), f64(W.v[idx, :heads])
    g = f64(W.g[:heads]) if W.gate == 0 else f64(W.g[idx, :heads])
    beta = None if W.beta is None else f64(W.beta[idx, :heads])
    t0 = time.perf_counter()
    oracle.segment_build(k, v, g, beta, ends - lens, ends, gate=W.gate, delta=W.delta)
    dt = time.perf_counter() - t0
    tok = int(lens.sum())
    rate = tok * heads / W.n_heads / dt   # tokens/s over all heads of the layer
    return {"value": round(rate, 1), "unit": "tokens/s", "cores": n_thr, "kind": "oracle",
            "sample": f"fp64 token-recurrence build of {len(segs)} of the workload's segments ({tok} tokens) "
                      f"x {heads} of {W.n_heads} heads in {dt:.2f} s, scaled to all heads"}


if __name__ == "__main__":
    sys.exit(main())
