#!/usr/bin/env python3
"""Benchmark of the HYPIC linear-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--only]
                    [--no-cpu-baseline] [--calibrate-copy MIB]

One step = one pass of the hot path over one synthetic batch with all inputs resident
in HBM.  The headline workload (default) is the largest one:

* kda-32h-d128-131k: 64 segments x 2048 tokens of a KDA-style layer (32 heads, d = 128,
  bf16, per-channel gate) are built (T_C, S(C|0)) with T cached as bf16 hi/lo planes,
  then 64 requests each compose 256 cached segments per layer for 30 layers (one
  composition call over 1920 chains; the 30 per-layer caches are distinct copies).

Besides it, unless --only: the same workload's stress variant (T_C of order one, so no
transition work underflows), and the 100,000-token gated-DeltaNet prompt
gdn-16h-d128-100k-seam (26 cold segments built, then one seam-advance call stepping the
127 w = 8 seam windows and composing all 128 pairs in order) with its stress variant and
the fused cold prefill.

Prints one JSON line.  `value` is segment-build tokens/s (tokens built per second of
build time); `compose_us_per_segment` is the composition time per (request, segment,
layer) with all heads.  Every library call is timed with HIP events on the stream it is
launched on.  `roofline` is for the call with the largest share of the headline step:
t_roof = max(F_alg / P_mfma, B / BW), with B the counter-measured HBM bytes of that call
where a stored measurement matches the current kernel sources, else its algorithmic
bytes; `frac` = t_roof / t_measured.  `cpu_baseline` times the fp64 oracle (test
infrastructure) on a bounded sample of the headline workload.
"""
from __future__ import annotations

import argparse
import ctypes
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 / fp16 MFMA, the precision the kernels multiply in
METRIC = "segment-build tokens/s + compose µs/segment on 1 GPU, % of MFMA/HBM roofline"
HEADLINE = "kda-32h-d128-131k"
SECONDARY = [("kda-32h-d128-131k", True), ("gdn-16h-d128-100k-seam", False), ("gdn-16h-d128-100k-seam", True)]
WORKLOADS = ["retnet-8h-d64", "gdn-16h-d128-32k", "gdn-16h-d128-100k-seam", "kda-32h-d128-131k"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=HEADLINE, choices=WORKLOADS)
    p.add_argument("--stress", action="store_true", help="the workload's stress variant")
    p.add_argument("--only", action="store_true", help="the chosen workload only (no secondary workloads)")
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

    def avg(self, name):
        return self.totals[name] / self.counts[name]


def roofline(flops, bytes_, t, traffic=None):
    """t_roof = max(F / P, B / BW), B the measured HBM bytes when given (L2 <-> fabric
    traffic from FETCH_SIZE + WRITE_SIZE), else the algorithmic bytes; the binding roof, the
    rate achieved against it (with that same B) and the fractions of both roofs."""
    b = traffic if traffic is not None else bytes_
    t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    t_hbm = b / (HBM_PEAK_GBS * 1e9)
    if t_mfma >= t_hbm:
        r = {"bound": "mfma", "achieved": round(flops / t / 1e12, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
             "unit": "TFLOP/s"}
    else:
        r = {"bound": "hbm", "achieved": round(b / t / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "bytes": "measured" if traffic is not None else "algorithmic"}
    r["frac"] = round(max(t_mfma, t_hbm) / t, 4)
    r["mfma_frac"] = round(t_mfma / t, 4)
    r["hbm_frac"] = round(t_hbm / t, 4)
    return r


def run_workload(torch, name, stress, steps, warmup, rotate=2, calibrate_copy=0, prefill=True):
    """Runs one workload's step `warmup` + `steps` times; returns its result dict."""
    from hybrid_attention_prefill_amd import binding as hb
    from hybrid_attention_prefill_amd import workloads as wl

    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    W = wl.make(name, stress=stress)
    t_gen = time.perf_counter() - t_gen
    seam_plan = W.seam_start is not None
    layered = W.n_layers > 1
    H, d = W.n_heads, W.d_k
    dt = torch.bfloat16 if W.in_dtype == "bf16" else torch.float32
    T = lambda a, t: torch.from_numpy(np.ascontiguousarray(a)).to(device=dev, dtype=t)
    in_bytes = 2 if W.in_dtype == "bf16" else 4
    gate_elems = {0: 0, 1: 1, 2: d}[W.gate]
    # constant decay caches T as one number; dense T is cached in the composition kernels'
    # operand format (bf16 hi/lo planes, 4 bytes per entry like fp32)
    t_layout = hb.T_SCALAR if W.gate == hb.GATE_HEAD else hb.T_SPLIT
    tsz = 1 if t_layout == hb.T_SCALAR else d * d
    tdt = torch.bfloat16 if t_layout == hb.T_SPLIT else torch.float32
    tshape = lambda n: (n, H) if t_layout == hb.T_SCALAR else (n, H, 2, d * d)
    per_tok = H * ((2 * d + gate_elems + (1 if W.delta else 0)) * in_bytes)   # k, v, gate, beta per token

    def inputs():
        x = dict(k=T(W.k, dt), v=T(W.v, dt), g=T(W.g, torch.float32 if W.gate == 0 else dt))
        x["beta"] = T(W.beta, dt) if W.beta is not None else None
        x["q"] = T(W.q, dt) if (W.q is not None and seam_plan) else None
        return x

    # Inputs that fit the 256 MB MALL several times over are kept in `rotate` copies, one per
    # step in turn, so a step never reads what the previous one left in the MALL.
    input_bytes = W.n_tokens * per_tok
    n_copies = 1 if input_bytes >= (1 << 30) else rotate
    X = [inputs() for _ in range(n_copies)]

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
        n_warm = len(warm)
        sb_all, se_all = T(W.cache_begin[order], torch.int64), T(W.cache_end[order], torch.int64)
        caches = []
        for x in X:   # one pair cache per input copy; warm pairs from an untimed earlier build
            Tc = torch.empty(tshape(W.n_seg), device=dev, dtype=tdt)
            Sc = torch.empty((W.n_seg, H, d, d), device=dev)
            hb.segment_build(x["k"], x["v"], x["g"], x["beta"], sb_all, se_all, gate=W.gate, delta=W.delta,
                             t_layout=t_layout, T_out=Tc, S_out=Sc)
            caches.append((Tc, Sc))
        sb_c, se_c = T(W.cache_begin[cold], torch.int64), T(W.cache_end[cold], torch.int64)
        ids = T(slot[None, :], torch.int32)
        seam = T(W.seam_start, torch.int64)
        R = torch.zeros((1, H, d, d), device=dev)
        out = torch.zeros((1, W.n_seg, W.w, H, d), device=dev)
        ws = torch.empty(hb.seam_workspace_bytes(H, d, d, 1, W.n_seg, W.w), device=dev, dtype=torch.uint8)
        wsb = build_workspace(len(cold))
        cold_tokens = int((W.cache_end[cold] - W.cache_begin[cold]).sum())

        def step(i):
            x = X[i % n_copies]
            Tc, Sc = caches[i % n_copies]
            timer.run("segment_build", lambda: hb.segment_build(x["k"], x["v"], x["g"], x["beta"], sb_c, se_c,
                                                                gate=W.gate, delta=W.delta, t_layout=t_layout,
                                                                T_out=Tc[n_warm:], S_out=Sc[n_warm:],
                                                                workspace=wsb))
            R.zero_()
            timer.run("seam_advance", lambda: hb.seam_advance(x["q"], x["k"], x["v"], x["g"], x["beta"], seam, R,
                                                              out, gate=W.gate, delta=W.delta, w=W.w,
                                                              scale=W.scale, pair_id=ids, T_cache=Tc, S_cache=Sc,
                                                              workspace=ws))

        built_tokens = cold_tokens
        prefill_segs = (sb_c, se_c)
        n_segments_composed = W.n_seg
        n_windows = int((W.seam_start >= 0).sum())
        pair_bytes = W.n_seg * H * (tsz + d * d) * 4
        work = {
            "segment_build": dict(bytes=cold_tokens * per_tok + len(cold) * H * (tsz + d * d) * 4,
                                  flops=cold_tokens * H * 4 * d * (d + d)),
            "seam_advance": dict(
                bytes=pair_bytes + n_windows * W.w * H * ((3 * d + 2) * in_bytes + d * 4),
                flops=W.n_seg * H * 2 * d * d * d + n_windows * W.w * H * 6 * d * d),
        }
        info.update(cold_segments=int(len(cold)), cold_tokens=cold_tokens, seam_windows=n_windows, w=W.w)
    else:
        sb, se = T(W.cache_begin, torch.int64), T(W.cache_end, torch.int64)
        n_chain, n_step = W.pair_id.shape
        ids = T(W.pair_id, torch.int32)
        built_tokens = int((W.cache_end - W.cache_begin).sum())
        prefill_segs = (sb, se)
        builds = [(torch.empty(tshape(W.n_seg), device=dev, dtype=tdt), torch.empty((W.n_seg, H, d, d), device=dev))
                  for _ in X]
        if layered:
            # one distinct cache copy per layer (so re-reads of a layer's pairs cannot come
            # from the MALL across layers): copies of one untimed earlier build
            Tb, Sb = builds[0]
            x = X[0]
            hb.segment_build(x["k"], x["v"], x["g"], x["beta"], sb, se, gate=W.gate, delta=W.delta,
                             t_layout=t_layout, T_out=Tb, S_out=Sb)
            Tc = Tb.repeat(W.n_layers, *([1] * (Tb.dim() - 1)))
            Sc = Sb.repeat(W.n_layers, 1, 1, 1)
            caches = [(Tc, Sc)] * len(X)
        else:
            caches = builds
        R = torch.zeros((n_chain, H, d, d), device=dev)
        wsb = build_workspace(W.n_seg)

        def step(i):
            x = X[i % n_copies]
            Tb, Sb = builds[i % n_copies]
            Tc, Sc = caches[i % n_copies]
            timer.run("segment_build", lambda: hb.segment_build(x["k"], x["v"], x["g"], x["beta"], sb, se,
                                                                gate=W.gate, delta=W.delta, t_layout=t_layout,
                                                                T_out=Tb, S_out=Sb, workspace=wsb))
            R.zero_()
            timer.run("compose", lambda: hb.compose(Tc, Sc, ids, R, t_layout=t_layout))

        n_segments_composed = n_chain * n_step
        used = np.unique(W.pair_id[W.pair_id >= 0])
        work = {
            "segment_build": dict(
                bytes=built_tokens * per_tok + W.n_seg * H * (tsz + d * d) * 4,
                flops=built_tokens * H * (2 * d * d if W.gate == hb.GATE_HEAD else 4 * d * (d + d))),
            # compose: every distinct pair read once and the running states read and written
            # once (the traffic floor); per reference: every step's pair read from HBM
            "compose": dict(bytes=len(used) * H * (tsz + d * d) * 4 + n_chain * H * d * d * 4 * 2,
                            bytes_per_reference=n_segments_composed * H * (tsz + d * d) * 4,
                            flops=n_segments_composed * H * (2 * d * d if tsz == 1 else 2 * d * d * d)),
        }
        info.update(segments=W.n_seg, built_tokens=built_tokens, chains=n_chain, steps_per_chain=n_step,
                    layers=W.n_layers)

    if calibrate_copy > 0:
        n = calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    timer.reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timer.collect()

    # After the timed steps: the fused cold prefill of the same (built) segments, with and
    # without T -- T's share of the linear layer's prefill on these segments (outputs need
    # each token's prefix state, so these segments are not cut).
    pf = None
    if prefill and W.gate == hb.GATE_TOKEN and W.delta and W.in_dtype == "bf16" and d in (64, 128) and W.q is not None:
        x = X[0]
        if x["q"] is None:
            x["q"] = T(W.q, dt)
        pb, pe = prefill_segs
        n_pf = pb.shape[0]
        pout = torch.empty((W.n_tokens, H, d), device=dev)
        pS = torch.empty((n_pf, H, d, d), device=dev)
        pT = torch.empty(tshape(n_pf), device=dev, dtype=tdt)
        calls = {
            "with_T": lambda: hb.segment_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], pb, pe, scale=W.scale,
                                                 t_layout=t_layout, T_out=pT, S_out=pS, out=pout),
            "S_only": lambda: hb.segment_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], pb, pe, scale=W.scale,
                                                 want_T=False, S_out=pS, out=pout),
        }
        ptimer = Timer(torch)
        for _ in range(2):
            for fn in calls.values():
                fn()
        torch.cuda.synchronize()
        for _ in range(max(3, min(steps, 10))):
            for nm, fn in calls.items():
                ptimer.run(nm, fn)
        ptimer.collect()
        pt = {nm: ptimer.avg(nm) for nm in calls}
        pf = {"with_T_us": round(pt["with_T"] * 1e6, 2), "S_only_us": round(pt["S_only"] * 1e6, 2),
              "T_overhead": round(pt["with_T"] / pt["S_only"] - 1, 4),
              "tokens_per_s_with_T": round(built_tokens / pt["with_T"], 1)}

    kern = {}
    for nm in timer.totals:
        avg = timer.avg(nm)
        wk = work[nm]
        traffic = measured_traffic(W.name, nm)
        k = dict(avg_us=round(avg * 1e6, 2), alg_bytes=int(wk["bytes"]), alg_flops=int(wk["flops"]),
                 GBps=round(wk["bytes"] / avg / 1e9, 1), TFLOPps=round(wk["flops"] / avg / 1e12, 2),
                 traffic=traffic, roofline=roofline(wk["flops"], wk["bytes"], avg, traffic))
        if "bytes_per_reference" in wk:
            k["bytes_per_reference"] = int(wk["bytes_per_reference"])
            k["GBps_per_reference"] = round(wk["bytes_per_reference"] / avg / 1e9, 1)
        kern[nm] = k
    build_avg = timer.avg("segment_build")
    chain_name = "seam_advance" if "seam_advance" in kern else "compose"
    chain_avg = timer.avg(chain_name)
    res = {
        "workload": W.name, "heads": H, "d_k": d, "d_v": d,
        "t_cache": {hb.T_SCALAR: "scalar f32", hb.T_SPLIT: "bf16 hi/lo planes"}[t_layout], **info,
        "input_copies": n_copies, "generate_s": round(t_gen, 1),
        "build_tokens_per_s": round(built_tokens / build_avg, 1),
        "build_us": round(build_avg * 1e6, 2),
        "compose_us_per_segment": round(chain_avg / n_segments_composed * 1e6, 4),
        "ms_per_step": round(wall / steps * 1e3, 4),
        "steps": steps,
        "kernels": kern,
    }
    if pf is not None:
        res["prefill"] = pf
    del X, caches, R
    if not seam_plan:
        del builds
    return res, W


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU path is not part "
              "of this build.", file=sys.stderr)
        return 1
    import torch

    torch.cuda.set_device(torch.device("cuda:0"))
    head, W = run_workload(torch, args.workload, args.stress, args.steps, args.warmup,
                           calibrate_copy=args.calibrate_copy)
    # the call with the largest share of the step
    dom = max(head["kernels"], key=lambda n: head["kernels"][n]["avg_us"])
    dk = head["kernels"][dom]
    roof = dict(dk["roofline"])
    roof.update(traffic=dk["traffic"], kernel=dom)
    line = {
        "metric": METRIC,
        "value": head["build_tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {k: head[k] for k in head if k not in ("kernels", "ms_per_step", "steps", "build_tokens_per_s",
                                                          "build_us", "compose_us_per_segment", "prefill")},
        "compose_us_per_segment": head["compose_us_per_segment"],
        "build_us": head["build_us"],
        "kernels": head["kernels"],
        "roofline": roof,
    }
    if "prefill" in head:
        line["prefill"] = head["prefill"]
    if not args.only:
        others = {}
        gc.collect()
        torch.cuda.empty_cache()
        for name, stress in SECONDARY:
            if (name, stress) == (args.workload, args.stress):
                continue
            r, _ = run_workload(torch, name, stress, max(3, min(args.steps, 10)), max(1, min(args.warmup, 2)),
                                prefill=not stress)
            others[r["workload"]] = r
            gc.collect()
            torch.cuda.empty_cache()
        line["workloads"] = others
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(W)
    print(json.dumps(line), flush=True)
    return 0


# Sources of the kernels each library call launches (a stored counter measurement is
# reported only while these files are unchanged); a segment build launches the kernels of
# its workload's transition family only.
BUILD_SOURCES = {"kda": ["build_kda.hip"], "gdn": ["build_gdn.hip", "build_split.hip"]}
CALL_SOURCES = {
    "seam_advance": ["seam.hip", "seam_chain.hip", "seam_layout.h", "compose.hip", "hypic_device.h", "hypic_kernels.h"],
    "compose": ["compose.hip", "hypic_device.h", "hypic_kernels.h"],
    "segment_build": ["build_gdn.hip", "build_split.hip", "build_kda.hip", "build_decay.hip", "build_common.h",
                      "hypic_device.h", "hypic_kernels.h"],
    "prefill_with_T": ["build_gdn.hip", "build_common.h", "hypic_device.h", "hypic_kernels.h"],
    "prefill_S_only": ["build_gdn.hip", "build_common.h", "hypic_device.h", "hypic_kernels.h"],
}


def call_sources(call, workload):
    fam = workload.split("-")[0]
    if call == "segment_build" and fam in BUILD_SOURCES:
        return BUILD_SOURCES[fam] + ["build_common.h", "hypic_device.h", "hypic_kernels.h"]
    return CALL_SOURCES[call]


def sources_digest(call, workload):
    import hashlib
    h = hashlib.sha256()
    for f in call_sources(call, workload):
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
                if rec.get("call") == call and rec.get("sources") == sources_digest(call, workload):
                    return int(rec["bytes_per_call"])
    return None


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(W):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload, packed and
    converted to fp64 before the clock starts: the build of some of its segments and the
    composition of a few of its chains (all heads), each also for one (segment, head) /
    (chain, head) unit, which runs on one thread."""
    import oracle
    n_thr = oracle.num_threads()
    pool = np.arange(W.n_seg)
    segs = {"retnet-8h-d64": pool, "gdn-16h-d128-32k": pool[:24], "gdn-16h-d128-100k-seam": pool,
            "kda-32h-d128-131k": pool[:8]}[W.name.replace("-stress", "")]
    heads = W.n_heads
    parts = [np.arange(W.cache_begin[s], W.cache_end[s]) for s in segs]
    idx = np.concatenate(parts)
    lens = np.array([len(p) for p in parts])
    ends = np.cumsum(lens)
    f64 = lambda a: np.ascontiguousarray(a, dtype=np.float64)
    k, v = f64(W.k[idx, :heads]), f64(W.v[idx, :heads])
    g = f64(W.g[:heads]) if W.gate == 0 else f64(W.g[idx, :heads])
    beta = None if W.beta is None else f64(W.beta[idx, :heads])
    t0 = time.perf_counter()
    T, S = oracle.segment_build(k, v, g, beta, ends - lens, ends, gate=W.gate, delta=W.delta)
    dt = time.perf_counter() - t0
    tok = int(lens.sum())
    rate = tok * heads / W.n_heads / dt   # tokens/s over all heads of the layer
    # one (segment, head): one unit, so one thread
    L0 = int(lens[0])
    t0 = time.perf_counter()
    oracle.segment_build(k[:L0, :1], v[:L0, :1], g[:1] if W.gate == 0 else g[:L0, :1],
                         None if beta is None else beta[:L0, :1], [0], [L0], gate=W.gate, delta=W.delta)
    dt1 = time.perf_counter() - t0
    out = {"value": round(rate, 1), "unit": "tokens/s", "cores": n_thr, "kind": "oracle",
           "cpu_model": _cpu_model(),
           "sample": f"fp64 token-recurrence build of {len(segs)} of the workload's segments ({tok} tokens) "
                     f"x {heads} of {W.n_heads} heads in {dt:.2f} s, scaled to all heads",
           "single_thread_build_tokens_per_s": round(L0 / dt1 / W.n_heads, 1)}
    # composition: a few chains of the plan with the pairs just built (T dense fp64)
    if W.pair_id is not None and W.pair_id.shape[1] > 1:
        n_seg_s = len(segs)
        n_ch = min(4, W.pair_id.shape[0])
        ids = np.ascontiguousarray(W.pair_id[:n_ch] % W.n_seg % n_seg_s, dtype=np.int32)
        Tc = T if T is not None else np.broadcast_to(np.eye(W.d_k), S.shape[:2] + (W.d_k, W.d_k)).copy()
        if heads < W.n_heads:
            reps = -(-W.n_heads // heads)
            Tc = np.tile(Tc, (1, reps, 1, 1))[:, :W.n_heads]
            Sc = np.tile(S, (1, reps, 1, 1))[:, :W.n_heads]
        else:
            Sc = S
        Tc, Sc = np.ascontiguousarray(Tc), np.ascontiguousarray(Sc)
        t0 = time.perf_counter()
        oracle.compose(Tc, Sc, ids)
        dtc = time.perf_counter() - t0
        n_steps = int((ids >= 0).sum())
        out["compose_us_per_segment"] = round(dtc / n_steps * 1e6, 2)
        out["compose_sample"] = (f"fp64 composition of {n_ch} chains x {ids.shape[1]} steps x {W.n_heads} heads "
                                 f"in {dtc:.2f} s")
        t0 = time.perf_counter()
        oracle.compose(Tc[:, :1], Sc[:, :1], ids[:1, :64])
        dt1 = time.perf_counter() - t0
        out["single_thread_compose_us_per_segment"] = round(dt1 / int((ids[0, :64] >= 0).sum()) * W.n_heads * 1e6, 2)
    return out


if __name__ == "__main__":
    sys.exit(main())
