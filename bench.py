#!/usr/bin/env python3
"""Bench of the gated residual add and the RMSNorm modulation on one MI355X.

One step is one pass of the whole path over the workload resident in HBM:
  1. gated residual add, full gate,  [1, 8160, 4096]           (out-of-place)
  2. gated residual add, bcast gate, [1, 32640, 4096]          (in place on x)
  3. rms_modulate,                   [2, 32640, 4096] -> y
  4. gated residual add, bcast gate, [2, 32640, 4096]          (in place on x)
Steps 1 and 2 are the two shapes the headline metric names (the
ltx2_full_s8160_c4096 and ltx2_bcast_s32640_c4096 workloads of the
residual-gate page's kernel benchmark); steps 3-4 are the modulation then the
gated residual of one DiT block at B = 2 (video hidden 4096).

Reported (one JSON line on stdout):
  value        algorithmic bytes of one step / measured time of one step, GB/s
  per_launch   per-call microseconds and GB/s from HIP events recorded on the
               launch stream around every call of the timed steps (timing-only
               events without the system-scope cache fence)
  cold         per-call microseconds with the caches flushed before each call
               (a 1 GiB read with cache-allocating loads pushes earlier data
               out of the L2s and the 256 MB memory-side cache and leaves
               only clean lines), median of repetitions; frac_of_hbm_peak
               and frac_of_mix_ceiling of every launch come from it
  mix_ceilings the read:write mixes of the step's launches on their own
               (rga_stream: the gate-add kernels' access shape with an XOR for
               arithmetic), timed by the same cold protocol on buffers of the
               launches' sizes: 3 reads + 1 write at [1,8160,4096] (c3's mix),
               2 reads + 1 write in place at [1,32640,4096] (c4's) and at
               [2,32640,4096] (c5's gate-add), 1 read + 1 write at
               [2,32640,4096] (the modulation's), and a read-only stream
  small_configs the other workload configurations (c1 full [1,126,2048] +
               rms_modulate, c2 bcast [1,L,3072] for L = 512, 4096, 4608):
               cold per-call time, and back-to-back per-call time (launch
               overhead and cache-resident inputs dominate at these sizes)
  variants     a compact set by default (the ideogram4 [1,4096,4608] bcast
               shape, binary16 rms_modulate and bf16 LayerNorm modulation at
               [2,32640,4096], the tanh-GELU on the FFN intermediate
               [1,32640,16384]); with --variants 1 every _ex variant as
               well (binary16 and binary32 storage, per-token modulation, the
               element-wise paths for ragged D, element offsets and rows past
               the register limit); cold and back-to-back per-call time
  ablations    with --ablations 1: the broadcast-gate add at c4 in the
               shapes the library does not use (rows per wave with the gate
               held, store cache policies), cold, and the store policies
               inside a chain of kernels on rotating buffers
  fused        the residual update + next modulation fused into one pass
               (rga_gate_add_rms_modulate) at the [2,32640,4096] shapes,
               back to back against the step's own separate launches of the
               two kernels, and cold (each call after the 1 GiB read)
  roofline     the kernel with the largest share of the step's time, against
               the 8 TB/s HBM peak
  cpu_baseline the CPU oracle on the same workload on this host's cores
Algorithmic bytes: each input element read once and each output element
written once, 2 bytes per element; a broadcast row counts once per call.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("achieved HBM GB/s and µs/call at [1,32640,4096] bcast and "
          "[1,8160,4096] full")
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class HipEvents:
    """Timing events straight from the HIP runtime that torch loaded (same
    SONAME, so dlopen returns torch's copy), created with
    hipEventDisableSystemFence: recording them does not write back and
    invalidate the caches the way default timing events do, which otherwise
    adds microseconds to every bracketed launch and cools the next one."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []

    def _check(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def new(self):
        ev = self.ct.c_void_p()
        self._check(self.hip.hipEventCreateWithFlags(self.ct.byref(ev), HIP_EVENT_DISABLE_SYSTEM_FENCE),
                    "hipEventCreateWithFlags")
        self.events.append(ev)
        return ev

    def record(self, ev, stream):
        self._check(self.hip.hipEventRecord(ev, self.ct.c_void_p(stream.cuda_stream)), "hipEventRecord")

    def sync(self, ev):
        self._check(self.hip.hipEventSynchronize(ev), "hipEventSynchronize")

    def ms(self, a, b):
        out = self.ct.c_float()
        self._check(self.hip.hipEventElapsedTime(self.ct.byref(out), a, b), "hipEventElapsedTime")
        return out.value

    def close(self):
        for ev in self.events:
            self.hip.hipEventDestroy(ev)
        self.events = []
HBM_PEAK_GBPS = 8000.0
FLUSH_BYTES = 1 << 30


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--cold-reps", type=int, default=30,
                   help="repetitions per launch of the cache-flushed timing (0: skip)")
    p.add_argument("--cpu-fraction", type=float, default=1.0,
                   help="fraction of each launch's rows the CPU oracle runs on (0: skip)")
    p.add_argument("--small-configs", type=int, default=1,
                   help="1: also time the c1/c2 configurations (0: skip)")
    p.add_argument("--variants", type=int, default=0,
                   help="0: the compact variant set; 1: every _ex variant as well "
                        "(storage types, per-token modulation, element-wise paths); "
                        "-1: none")
    p.add_argument("--mix-ceilings", type=int, default=1,
                   help="1: time the read:write mix ceilings of the step's launches")
    p.add_argument("--ablations", type=int, default=0,
                   help="1: time the broadcast-gate add in the shapes the library does "
                        "not use (row tiles, store policies)")
    p.add_argument("--fused-reps", type=int, default=30,
                   help="repetitions of the fused-vs-separate comparison (0: skip)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="repeat the CPU oracle sample until this much time has passed")
    p.add_argument("--summarize", nargs="+", metavar="ARG",
                   help="no GPU run: summarize rocprofv3 csv output of this bench. "
                        "'trace KERNEL_TRACE.csv [BENCH.json]' prints per-launch-shape "
                        "device durations; 'counters OUT.json CSV...' prints HBM bytes "
                        "(FETCH_SIZE, WRITE_SIZE scaled by the 1 GiB copy) and instruction "
                        "counts per launch shape and writes the traffic summary OUT.json; "
                        "'variants BENCH.json CSV...' prints per-variant kernels and device "
                        "times (kernel trace) or HBM bytes and instruction counts (counter "
                        "files) for a run with --variants 1 --fused-reps 0 --ablations 0")
    return p.parse_args()


def main():
    args = parse_args()
    if args.summarize:
        summarize(args.summarize)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this path runs on one GPU only (asked for {max(args.gpus, world)}); "
              "the workload is row-local and would shard over tokens with no exchange, "
              "but multi-GPU runs are not part of this build.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import __graft_entry__
    __graft_entry__._ensure_built()
    import diffusion_transformer_elementwise_amd as dte
    from synth_inputs import CASES, GATE_BCAST, GATE_FULL, make_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    def to_dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    log = lambda m: print(f"[bench] {m}", file=sys.stderr, flush=True)

    c3, c4, c5 = CASES["c3"], CASES["c4"], CASES["c5"]
    log("generating seeded inputs (c3, c4, c5)")
    host = {k: make_inputs(CASES[k]) for k in ("c3", "c4", "c5")}
    d3 = {k: to_dev(v) for k, v in host["c3"].items()}
    d4 = {k: to_dev(v) for k, v in host["c4"].items()}
    d5 = {k: to_dev(v) for k, v in host["c5"].items()}
    out3 = torch.empty_like(d3["x"])
    y5 = torch.empty_like(d5["x"])
    if args.cpu_fraction <= 0:
        host = None

    def gate_bytes(c):
        return (4 * c.elems if c.gate == GATE_FULL else 3 * c.elems + c.B * c.D) * 2

    launches = [
        ("c3_full_gate_add", "gate_add_full_kernel", gate_bytes(c3),
         lambda: dte.rga_residual_gate_add(d3["x"], d3["u"], d3["g"], out=out3, gate_mode=GATE_FULL)),
        ("c4_bcast_gate_add_inplace", "gate_add_bcast_kernel", gate_bytes(c4),
         lambda: dte.rga_residual_gate_add(d4["x"], d4["u"], d4["g"], out=d4["x"], gate_mode=GATE_BCAST)),
        ("c5_rms_modulate", "rms_modulate_kernel", (2 * c5.elems + 2 * c5.B * c5.D) * 2,
         lambda: dte.rms_modulate(d5["x"], d5["scale"], d5["shift"], c5.eps, out=y5)),
        ("c5_bcast_gate_add_inplace", "gate_add_bcast_kernel", gate_bytes(c5),
         lambda: dte.rga_residual_gate_add(d5["x"], d5["u"], d5["g"], out=d5["x"], gate_mode=GATE_BCAST)),
    ]
    step_bytes = sum(l[2] for l in launches)

    # copy ceiling on 1 GiB (also the known-size kernel for counter scaling)
    src = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    dte.fill_(src, 0x3F803F80)
    dte.copy_(dst, src)
    torch.cuda.synchronize()
    hev = HipEvents()
    ev = [hev.new() for _ in range(2)]
    hev.record(ev[0], stream)
    for _ in range(10):
        dte.copy_(dst, src)
    hev.record(ev[1], stream)
    torch.cuda.synchronize()
    copy_gbps = 10 * 2 * FLUSH_BYTES / (hev.ms(ev[0], ev[1]) * 1e-3) / 1e9
    log(f"copy ceiling {copy_gbps:.0f} GB/s")
    # the cache flush's own rate: cache-allocating loads, not a ceiling
    hev.record(ev[0], stream)
    for _ in range(10):
        dte.read_(src, sink)
    hev.record(ev[1], stream)
    torch.cuda.synchronize()
    flush_gbps = 10 * FLUSH_BYTES / (hev.ms(ev[0], ev[1]) * 1e-3) / 1e9
    log(f"flush read {flush_gbps:.0f} GB/s")
    del dst
    torch.cuda.empty_cache()

    e0, e1 = hev.new(), hev.new()

    def cold_times(fn, reps, before=None):
        """Per-call microseconds, each call after a 1 GiB cache-allocating read
        (and after `before`, untimed, when given)."""
        ts = []
        for _ in range(reps):
            if before is not None:
                before()
            dte.read_(src, sink)
            hev.record(e0, stream)
            fn()
            hev.record(e1, stream)
            hev.sync(e1)
            ts.append(hev.ms(e0, e1) * 1e3)
        return ts

    def run_step(events=None):
        for i, l in enumerate(launches):
            if events is not None:
                hev.record(events[i], stream)
            l[3]()
        if events is not None:
            hev.record(events[len(launches)], stream)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    evs = [[hev.new() for _ in range(len(launches) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        run_step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    durations = {l[0]: [] for l in launches}
    for k in range(args.steps):
        for i, l in enumerate(launches):
            durations[l[0]].append(hev.ms(evs[k][i], evs[k][i + 1]) * 1e3)  # us
    gpu_step_ms = statistics.mean(
        hev.ms(evs[k][0], evs[k][-1]) for k in range(args.steps))

    per_launch = {}
    for name, kernel, nbytes, _ in launches:
        us = statistics.mean(durations[name])
        per_launch[name] = {
            "kernel": kernel, "bytes": nbytes, "us": round(us, 2),
            "us_median": round(statistics.median(durations[name]), 2),
            "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}

    # cold protocol: flush, then time one call, per launch
    cold = {}
    if args.cold_reps > 0:
        log(f"cold timing, {args.cold_reps} reps per launch")
        for name, kernel, nbytes, fn in launches:
            ts = cold_times(fn, args.cold_reps)
            med = statistics.median(ts)
            cold[name] = {"us_median": round(med, 2),
                          "us_p10": round(float(np.percentile(ts, 10)), 2),
                          "us_p90": round(float(np.percentile(ts, 90)), 2),
                          "GBps": round(nbytes / (med * 1e-6) / 1e9, 1),
                          "frac_of_hbm_peak": round(nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}

    # the read:write mix of each launch on its own, same buffer sizes, same protocol
    mixes = {}
    if args.mix_ceilings and args.cold_reps > 0:
        log("mix ceilings")
        mixes = mix_ceilings(dte, torch, dev, cold_times, args.cold_reps, log)
        for name, m in mixes.items():
            for launch in m.get("compares_with", []):
                if launch in cold and m["cold_us_median"] < cold[launch].get(
                        "mix_ceiling_us", float("inf")):
                    cold[launch]["mix"] = name
                    cold[launch]["mix_ceiling_us"] = m["cold_us_median"]
                    cold[launch]["frac_of_mix_ceiling"] = round(
                        m["cold_us_median"] / cold[launch]["us_median"], 4)
        torch.cuda.empty_cache()

    def cold_and_warm(fn, nbytes, kernel):
        ts = cold_times(fn, args.cold_reps)
        hev.record(e0, stream)
        for _ in range(100):
            fn()
        hev.record(e1, stream)
        hev.sync(e1)
        warm = hev.ms(e0, e1) * 1e3 / 100
        med = statistics.median(ts)
        # the cold median is the measurement; back to back, inputs that fit
        # the 256 MB memory-side cache are served from it (context only)
        return {"kernel": kernel, "bytes": nbytes, "cold_reps": len(ts), "warm_reps": 100,
                "cold_us_median": round(med, 2),
                "cold_us_p10": round(float(np.percentile(ts, 10)), 2),
                "cold_us_p90": round(float(np.percentile(ts, 90)), 2),
                "cold_GBps": round(nbytes / (med * 1e-6) / 1e9, 1),
                "frac_of_hbm_peak": round(nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                "back_to_back_us": round(warm, 2),
                "back_to_back_GBps": round(nbytes / (warm * 1e-6) / 1e9, 1)}

    small = {}
    if args.small_configs and args.cold_reps > 0:
        log("small configs c1, c2")
        for key in ("c1", "c2a", "c2b", "c2c"):
            c = CASES[key]
            h = make_inputs(c)
            d = {k: to_dev(v) for k, v in h.items()}
            o = torch.empty_like(d["x"])
            small[c.name + "_gate_add"] = cold_and_warm(
                lambda: dte.rga_residual_gate_add(d["x"], d["u"], d["g"], out=o, gate_mode=c.gate),
                gate_bytes(c), "gate_add_full_kernel" if c.gate == GATE_FULL else "gate_add_bcast_kernel")
            small[c.name + "_gate_add"]["shape"] = [c.B, c.L, c.D]
            if c.rms:
                small[c.name + "_rms_modulate"] = cold_and_warm(
                    lambda: dte.rms_modulate(d["x"], d["scale"], d["shift"], c.eps, out=o),
                    (2 * c.elems + 2 * c.B * c.D) * 2, "rms_modulate_kernel")
                small[c.name + "_rms_modulate"]["shape"] = [c.B, c.L, c.D]
            del d, o

    variants = {}
    if args.variants >= 0 and args.cold_reps > 0:
        log("variants" + (": every _ex variant" if args.variants else ": compact set"))
        variants = run_variants(dte, torch, dev, cold_and_warm, log, full=bool(args.variants))
        torch.cuda.empty_cache()

    ablations = {}
    if args.ablations and args.cold_reps > 0:
        log("ablations: broadcast-gate add shapes and store policies at c4")
        ablations = run_ablations(dte, torch, dev, d4, cold_times, hev, stream, args.cold_reps, log)
        ablations["occupancy"] = run_occupancy(dte, torch, dev, d4, cold_times, hev, stream,
                                               args.cold_reps, log)
        torch.cuda.empty_cache()
        ablations["schedules"] = run_schedules(dte, torch, dev, d4, cold_times, hev, stream,
                                               args.cold_reps, log)
        torch.cuda.empty_cache()
        ablations["line_offsets"] = run_line_offsets(dte, torch, dev, cold_times,
                                                     args.cold_reps, log)
        torch.cuda.empty_cache()

    fused = {}
    if args.fused_reps > 0:
        log(f"fused residual + modulation, {args.fused_reps} reps")
        n5 = c5.elems
        fused_bytes = (4 * n5 + c5.B * c5.D + 2 * c5.B * c5.D) * 2
        pair_bytes = gate_bytes(c5) + (2 * n5 + 2 * c5.B * c5.D) * 2
        # warm-up launches first (the first launch of a kernel also loads its
        # code object); then all reps enqueued back to back (a host sync per
        # rep would leave the stream idle and bill the host's submission
        # latency to the launch after it), read after one sync
        fn = lambda: dte.rga_gate_add_rms_modulate(
            d5["x"], d5["u"], d5["g"], d5["scale"], d5["shift"], c5.eps,
            x_out=d5["x"], y=y5, gate_mode=GATE_BCAST)
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        efs = [hev.new() for _ in range(args.fused_reps + 1)]
        for k in range(args.fused_reps):
            hev.record(efs[k], stream)
            fn()
        hev.record(efs[-1], stream)
        torch.cuda.synchronize()
        tf = [hev.ms(efs[k], efs[k + 1]) * 1e3 for k in range(args.fused_reps)]
        fus = statistics.mean(tf)
        # the same two steps as separate launches: the step's own c5 gate-add
        # and rms_modulate launches (same kernels, shapes and bytes)
        pair = per_launch["c5_bcast_gate_add_inplace"]["us"] + per_launch["c5_rms_modulate"]["us"]
        fused = {"shape": "[2,32640,4096] bcast gate, x_out in place",
                 "kernel": "gate_add_rms_modulate_staged_kernel",
                 "bytes": fused_bytes, "us": round(fus, 2),
                 "GBps": round(fused_bytes / (fus * 1e-6) / 1e9, 1),
                 "frac_of_hbm_peak": round(fused_bytes / (fus * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                 "separate_pair_bytes": pair_bytes,
                 "separate_pair_us": round(pair, 2),
                 "separate_pair_from": "per_launch c5_bcast_gate_add_inplace + c5_rms_modulate",
                 "speedup_vs_separate": round(pair / fus, 3)}
        if args.cold_reps > 0:
            # the cold protocol of the step's launches (each call after the
            # 1 GiB read), beside the back-to-back mean above
            tc = cold_times(fn, args.cold_reps)
            cm = statistics.median(tc)
            fused.update({"cold_us_median": round(cm, 2),
                          "cold_us_p10": round(float(np.percentile(tc, 10)), 2),
                          "cold_us_p90": round(float(np.percentile(tc, 90)), 2),
                          "cold_frac_of_hbm_peak": round(
                              fused_bytes / (cm * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)})

    # roofline of the kernel with the largest share of the step, from the
    # step's own launches (the other shapes above do not enter it)
    by_kernel = {}
    for name, kernel, nbytes, _ in launches:
        agg = by_kernel.setdefault(kernel, {"bytes": 0, "us": 0.0, "launches": 0})
        agg["bytes"] += nbytes
        agg["us"] += statistics.mean(durations[name])
        agg["launches"] += 1
    dom = max(by_kernel, key=lambda k: by_kernel[k]["us"])
    agg = by_kernel[dom]
    bytes_per_launch = agg["bytes"] / agg["launches"]
    avg_us = agg["us"] / agg["launches"]
    achieved = bytes_per_launch / (avg_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": load_traffic(dom),
                "bytes_per_launch": bytes_per_launch,
                "avg_launch_us": round(avg_us, 2),
                "launches_per_step": agg["launches"]}

    hev.close()
    cpu = None
    if host is not None:
        del d3, d4, d5, out3, y5, src
        torch.cuda.empty_cache()
        cpu = cpu_baseline(host, args.cpu_fraction, args.cpu_seconds, log)

    headline = {}
    for key, launch in (("bcast_[1,32640,4096]", "c4_bcast_gate_add_inplace"),
                        ("full_[1,8160,4096]", "c3_full_gate_add")):
        headline[key] = {k: per_launch[launch][k] for k in ("us", "GBps")}
        if launch in cold:
            headline[key]["cold_us"] = cold[launch]["us_median"]
            headline[key]["cold_GBps"] = cold[launch]["GBps"]
            headline[key]["cold_frac_of_hbm_peak"] = cold[launch]["frac_of_hbm_peak"]
            if "frac_of_mix_ceiling" in cold[launch]:
                headline[key]["mix"] = cold[launch]["mix"]
                headline[key]["cold_frac_of_mix_ceiling"] = cold[launch]["frac_of_mix_ceiling"]

    result = {
        "metric": METRIC,
        "value": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "io_dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "ltx2 DiT elementwise step: full gate-add [1,8160,4096]; "
                        "bcast gate-add in place [1,32640,4096]; rms_modulate + "
                        "bcast gate-add in place [2,32640,4096]",
            "step_bytes": step_bytes,
            "gpu_time_per_step_ms": round(gpu_step_ms, 4),
            "headline": headline,
        },
        "per_launch": per_launch,
        "cold": cold,
        "mix_ceilings": mixes,
        "small_configs": small,
        "variants": variants,
        "fused": fused,
        "ablations": ablations,
        "copy_ceiling_GBps": round(copy_gbps, 1),
        "flush_read_GBps": round(flush_gbps, 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def mix_ceilings(dte, torch, dev, cold_times, reps, log):
    """rga_stream at the step's read:write mixes and sizes, cold protocol,
    in the launches' own shape (one 16-byte word per lane per stream) and,
    for the two metric launches' mixes, with two words per lane. Each entry
    names the launches it bounds (compares_with); a launch's ceiling is the
    fastest of its entries."""
    import numpy as np
    e3 = 8160 * 4096 * 2          # bytes of one [1,8160,4096] bf16 tensor
    e4 = 32640 * 4096 * 2         # [1,32640,4096]
    e5 = 2 * e4                   # [2,32640,4096]
    specs = [
        # name, sources, write (None / "new" / "inplace"), bytes per stream, words/lane, bounds
        ("3R:1W [1,8160,4096]", 3, "new", e3, 1, ["c3_full_gate_add"]),
        ("3R:1W [1,8160,4096], 2 words per lane", 3, "new", e3, 2, ["c3_full_gate_add"]),
        ("2R:1W in place [1,32640,4096]", 2, "inplace", e4, 1, ["c4_bcast_gate_add_inplace"]),
        ("2R:1W in place [1,32640,4096], 2 words per lane", 2, "inplace", e4, 2,
         ["c4_bcast_gate_add_inplace"]),
        ("2R:1W in place [2,32640,4096]", 2, "inplace", e5, 1, ["c5_bcast_gate_add_inplace"]),
        ("1R:1W [2,32640,4096]", 1, "new", e5, 1, ["c5_rms_modulate"]),
        ("R [2,32640,4096], 1 word per lane", 1, None, e5, 1, []),
        ("R [2,32640,4096], 2 words per lane", 1, None, e5, 2, []),
    ]
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    out = {}
    for name, nsrc, write, nbytes, wpl, bounds in specs:
        srcs = [torch.empty(nbytes // 4, dtype=torch.int32, device=dev) for _ in range(nsrc)]
        for k, t in enumerate(srcs):
            dte.fill_(t, 0x3F803F80 + k)
        dst = None
        if write == "new":
            dst = torch.empty(nbytes // 4, dtype=torch.int32, device=dev)
        elif write == "inplace":
            dst = srcs[0]
        fn = lambda: dte.stream_(srcs, dst, words_per_lane=wpl, sink=sink)
        fn()
        ts = cold_times(fn, reps)
        med = statistics.median(ts)
        total = nbytes * (nsrc + (1 if dst is not None else 0))
        out[name] = {"reads": nsrc, "writes": 0 if dst is None else 1,
                     "in_place": write == "inplace", "words_per_lane": wpl,
                     "bytes": total, "cold_us_median": round(med, 2),
                     "cold_us_p10": round(float(np.percentile(ts, 10)), 2),
                     "cold_us_p90": round(float(np.percentile(ts, 90)), 2),
                     "GBps": round(total / (med * 1e-6) / 1e9, 1),
                     "frac_of_hbm_peak": round(total / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                     "compares_with": bounds}
        log(f"mix {name}: {med:.2f} us, {total / (med * 1e-6) / 1e9:.0f} GB/s")
        del srcs, dst
    return out


def run_occupancy(dte, torch, dev, d4, cold_times, hev, stream, reps, log):
    """The row-modulation kernels (two rows per workgroup, scale/shift staged
    in LDS) at a chosen number of workgroups per CU (rga_modulate_occupancy,
    rga_fused_occupancy; -1 = no cap, 0 = the library's rule): the modulation
    and the fused call at [2,32640,4096] (16-byte-pack kernels) and
    [2,32640,4100] (register-row element kernels), bf16. Timed cold (median
    after a 1 GiB cache-allocating read) and right after the c4 gate-add
    (mean of 10 pairs, HIP events around the variant)."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(4242)
    out = {}

    def draw(shape, std):
        return (torch.randn(shape, generator=gen, device=dev) * std).to(torch.bfloat16)

    def after_c4(fn):
        evs = [(hev.new(), hev.new()) for _ in range(10)]
        for a, b in evs:
            dte.rga_residual_gate_add(d4["x"], d4["u"], d4["g"], out=d4["x"], gate_mode=1)
            hev.record(a, stream)
            fn()
            hev.record(b, stream)
        torch.cuda.synchronize()
        return statistics.mean(hev.ms(a, b) * 1e3 for a, b in evs)

    for D in (4096, 4100):
        B, L = 2, 32640
        x, u = draw((B, L, D), 2.0), draw((B, L, D), 1.0)
        g, s, t = draw((B, 1, D), 0.1), draw((B, 1, D), 0.1), draw((B, 1, D), 0.1)
        y, xo = torch.empty_like(x), torch.empty_like(x)
        mb = (2 * B * L * D + 2 * B * D) * 2
        fb = (4 * B * L * D + 3 * B * D) * 2
        for w in (-1, 0, 4, 5, 6, 8, 12):
            for name, nbytes, fn in (
                    (f"rms_modulate [2,32640,{D}]", mb,
                     lambda: dte.modulate_occupancy(x, s, t, 1e-6, out=y, wg_per_cu=w)),
                    (f"fused bcast [2,32640,{D}]", fb,
                     lambda: dte.fused_occupancy(x, u, g, s, t, 1e-6, x_out=xo, y=y,
                                                 wg_per_cu=w))):
                fn()
                med = statistics.median(cold_times(fn, reps))
                pair = after_c4(fn)
                key = f"{name} wg_per_cu={w}"
                out[key] = {"bytes": nbytes, "cold_us_median": round(med, 2),
                            "cold_frac_of_hbm_peak": round(nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                            "after_c4_us": round(pair, 2)}
                log(f"occupancy {key}: cold {med:.2f} us, after c4 {pair:.2f} us")
        del x, u, g, s, t, y, xo
    return out


# bytes of the line-offset copies, one size per offset: not the flush size,
# so that each offset's dispatches (its own grid) stay apart from the
# calibration copy's and from the other offsets'
LINE_OFFSETS = (0, 16, 64, 112)


def line_copy_bytes(offset):
    return FLUSH_BYTES - 4096 - 1024 * LINE_OFFSETS.index(offset)


def run_line_offsets(dte, torch, dev, cold_times, reps, log):
    """A nontemporal copy of about 1 GiB (rga_copy, line_copy_bytes) with
    source and destination at the same byte offset from a 128-byte line: 0
    (every wave instruction covers whole lines) and 16, 64, 112 (every
    instruction straddles one line more). Cold calls in rounds over the
    offsets; the median per offset."""
    n0 = FLUSH_BYTES
    src = torch.empty(n0 + 256, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    assert src.data_ptr() % 128 == 0 and dst.data_ptr() % 128 == 0
    dte.fill_(src.view(torch.int32), 0x3F803F80)
    offs = LINE_OFFSETS
    fns = {o: (lambda o=o: dte.copy_(dst[o:o + line_copy_bytes(o)], src[o:o + line_copy_bytes(o)]))
           for o in offs}
    times = {o: [] for o in offs}
    for o in offs:
        fns[o]()
    for _ in range(reps):
        for o in offs:
            times[o] += cold_times(fns[o], 1)
    out = {}
    for o in offs:
        n = line_copy_bytes(o)
        med = statistics.median(times[o])
        gbps = 2 * n / (med * 1e-6) / 1e9
        out[f"copy at byte offset {o}"] = {"bytes": 2 * n, "cold_us_median": round(med, 2),
                                           "GBps": round(gbps, 1),
                                           "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
        log(f"line offset {o}: {med:.2f} us, {gbps:.0f} GB/s")
    del src, dst
    return out


SCHEDULES = ("library", "loads_first", "one_plus", "two_rows", "prefetch")


def run_schedules(dte, torch, dev, d4, cold_times, hev, stream, reps, log):
    """The staged row-modulation kernels in each schedule (rga_modulate_variant,
    rga_fused_variant; SCHED_* in order): the modulation and the fused call
    (broadcast gate, out of place) at [2,32640,4096] bf16. Cold calls (after
    a 1 GiB cache-allocating read) taken in rounds that visit every schedule
    once, so drift over the run touches all alike; the median per schedule.
    Then right after the c4 gate-add (mean of 10 pairs, HIP events)."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(4343)
    B, L, D = 2, 32640, 4096

    def draw(shape, std):
        return (torch.randn(shape, generator=gen, device=dev) * std).to(torch.bfloat16)

    x, u = draw((B, L, D), 2.0), draw((B, L, D), 1.0)
    g, sc, sh = draw((B, 1, D), 0.1), draw((B, 1, D), 0.1), draw((B, 1, D), 0.1)
    y, xo = torch.empty_like(x), torch.empty_like(x)
    mb = (2 * B * L * D + 2 * B * D) * 2
    fb = (4 * B * L * D + 3 * B * D) * 2

    def modulation(k):
        return lambda: dte.modulate_variant(x, sc, sh, 1e-6, out=y, schedule=k)

    def fused(k):
        return lambda: dte.fused_variant(x, u, g, sc, sh, 1e-6, x_out=xo, y=y, schedule=k)

    calls = []
    for k, name in enumerate(SCHEDULES):
        calls.append((f"rms_modulate [2,32640,4096] schedule={name}", mb, modulation(k)))
        calls.append((f"fused bcast [2,32640,4096] schedule={name}", fb, fused(k)))
    times = {n: [] for n, _, _ in calls}
    for _, _, fn in calls:
        fn()
    for _ in range(reps):
        for n, _, fn in calls:
            times[n] += cold_times(fn, 1)

    def after_c4(fn):
        evs = [(hev.new(), hev.new()) for _ in range(10)]
        for a, b in evs:
            dte.rga_residual_gate_add(d4["x"], d4["u"], d4["g"], out=d4["x"], gate_mode=1)
            hev.record(a, stream)
            fn()
            hev.record(b, stream)
        torch.cuda.synchronize()
        return statistics.mean(hev.ms(a, b) * 1e3 for a, b in evs)

    out = {}
    for n, nbytes, fn in calls:
        med = statistics.median(times[n])
        pair = after_c4(fn)
        out[n] = {"bytes": nbytes, "cold_us_median": round(med, 2),
                  "cold_frac_of_hbm_peak": round(nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                  "after_c4_us": round(pair, 2)}
        log(f"schedule {n}: cold {med:.2f} us, after c4 {pair:.2f} us")
    del x, u, y, xo
    return out


def run_ablations(dte, torch, dev, d4, cold_times, hev, stream, reps, log):
    """The c4 broadcast-gate add (in place, [1,32640,4096]) in the shapes and
    store policies the library does not use (rga_gate_add_variant), cold; and
    each store policy inside a chain that leaves nothing to reuse from the
    caches: the gate-add on one of four rotating (x, u) sets, then a 1 GiB
    nontemporal copy, repeated; per-kernel and chain time from HIP events."""
    B, L, D = 1, 32640, 4096
    nbytes = (3 * B * L * D + B * D) * 2
    x, u, g = d4["x"], d4["u"], d4["g"]
    pol = {"nt": dte.STORE_NT, "plain": dte.STORE_PLAIN, "device": dte.STORE_DEVICE}
    out = {"shape": [B, L, D], "bytes": nbytes, "cold": {}, "chain": {}}
    for T in (1, 2, 4, 8):
        for pname, sp in pol.items():
            if T != 1 and pname != "nt":
                continue
            fn = lambda: dte.gate_add_variant(x, u, g, out=x, rows_per_wave=T, store_policy=sp)
            fn()
            ts = cold_times(fn, reps)
            med = statistics.median(ts)
            key = f"rows_per_wave={T} store={pname}"
            out["cold"][key] = {"us_median": round(med, 2),
                                "GBps": round(nbytes / (med * 1e-6) / 1e9, 1),
                                "frac_of_hbm_peak": round(nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
            log(f"ablation {key}: {med:.2f} us")
    # chain on rotating buffers: nothing a kernel reads was touched by the
    # previous few kernels, so a store policy that parks lines in a cache
    # pays their write-back inside the chain
    sets = [(torch.empty_like(x), torch.empty_like(u)) for _ in range(4)]
    for xs, us_ in sets:
        xs.copy_(x)
        us_.copy_(u)
    csrc = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
    cdst = torch.empty_like(csrc)
    dte.fill_(csrc, 0x3F803F80)
    steps = 16
    for pname, sp in pol.items():
        evs = [hev.new() for _ in range(2 * steps + 1)]
        for k in range(4):
            xs, us_ = sets[k % 4]
            dte.gate_add_variant(xs, us_, g, out=xs, rows_per_wave=1, store_policy=sp)
            dte.copy_(cdst, csrc)
        torch.cuda.synchronize()
        for k in range(steps):
            xs, us_ = sets[k % 4]
            hev.record(evs[2 * k], stream)
            dte.gate_add_variant(xs, us_, g, out=xs, rows_per_wave=1, store_policy=sp)
            hev.record(evs[2 * k + 1], stream)
            dte.copy_(cdst, csrc)
        hev.record(evs[-1], stream)
        torch.cuda.synchronize()
        tg = statistics.mean(hev.ms(evs[2 * k], evs[2 * k + 1]) * 1e3 for k in range(steps))
        tc = statistics.mean(hev.ms(evs[2 * k + 1], evs[2 * k + 2]) * 1e3 for k in range(steps))
        out["chain"][f"store={pname}"] = {"gate_add_us": round(tg, 2), "copy_1GiB_us": round(tc, 2),
                                          "pair_us": round(tg + tc, 2)}
        log(f"ablation chain store={pname}: gate {tg:.2f} us, copy {tc:.2f} us")
    del sets, csrc, cdst
    return out


def run_variants(dte, torch, dev, cold_and_warm, log, full=False):
    """The _ex variants at DiT shapes, each timed cold (caches flushed) and
    back to back; with full=False only a compact set (ideogram4, binary16
    rms_modulate, bf16 LayerNorm modulation, bf16 tanh-GELU). Inputs: seeded normal draws on the device (x N(0,2), u
    N(0,1), gate uniform(-1,1), scale/shift N(0,0.1)), out of place.
    Algorithmic bytes: every input element read once (a broadcast row once
    per call), every output element written once, at the storage size."""
    from synth_inputs import EXTRA_CASES, make_inputs

    gen = torch.Generator(device=dev)
    gen.manual_seed(20240)
    T = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}

    def draw(shape, dt, std=1.0, uniform=False, offset=0):
        n = 1
        for v in shape:
            n *= v
        flat = torch.empty(n + offset, dtype=T[dt], device=dev)
        if uniform:
            a = torch.rand(n, generator=gen, device=dev) * 2 - 1
        else:
            a = torch.randn(n, generator=gen, device=dev) * std
        flat[offset:].copy_(a)
        return flat[offset:].view(shape)

    out = {}

    def gate(name, B, L, D, dt, mode, offset=0):
        x = draw((B, L, D), dt, 2.0, offset=offset)
        u = draw((B, L, D), dt, offset=offset)
        g = draw((B, L, D) if mode == dte.GATE_FULL else (B, 1, D), dt, uniform=True, offset=offset)
        o = draw((B, L, D), dt, offset=offset)
        es = x.element_size()
        n = B * L * D
        nbytes = (4 * n if mode == dte.GATE_FULL else 3 * n + B * D) * es
        fast = D % 8 == 0 and offset == 0
        fast = fast or (mode == dte.GATE_FULL and offset == 0)  # a full add is one flat stream
        kern = ("gate_add_full_kernel" if mode == dte.GATE_FULL else "gate_add_bcast_kernel") \
            if fast else ("gate_add_generic_full_kernel" if mode == dte.GATE_FULL
                          else "gate_add_generic_bcast_kernel")
        log(f"variant {name}")
        out[name] = cold_and_warm(lambda: dte.rga_residual_gate_add_ex(x, u, g, out=o),
                                  nbytes, kern)

    def rms(name, B, L, D, dt, mod, offset=0):
        mshape = (B, L, D) if mod == dte.MOD_TOKEN else (B, 1, D)
        x = draw((B, L, D), dt, 2.0, offset=offset)
        sc, sh = draw(mshape, dt, 0.1, offset=offset), draw(mshape, dt, 0.1, offset=offset)
        o = draw((B, L, D), dt, offset=offset)
        es = x.element_size()
        n = B * L * D
        nbytes = (2 * n + 2 * (n if mod == dte.MOD_TOKEN else B * D)) * es
        fast = D % 8 == 0 and offset == 0 and D <= dte.RGA_RMS_MAX_D
        log(f"variant {name}")
        out[name] = cold_and_warm(
            lambda: dte.rga_rms_modulate_ex(x, sc, sh, 1e-6, out=o, mod_mode=mod), nbytes,
            "rms_modulate_kernel" if fast else element_norm_kernel("rms", D, dt, mod))

    def fused(name, B, L, D, dt, mode, mod):
        mshape = (B, L, D) if mod == dte.MOD_TOKEN else (B, 1, D)
        x, u = draw((B, L, D), dt, 2.0), draw((B, L, D), dt)
        g = draw((B, L, D) if mode == dte.GATE_FULL else (B, 1, D), dt, uniform=True)
        sc, sh = draw(mshape, dt, 0.1), draw(mshape, dt, 0.1)
        xo, y = torch.empty_like(x), torch.empty_like(x)
        es = x.element_size()
        n = B * L * D
        nbytes = (4 * n + (n if mode == dte.GATE_FULL else B * D)
                  + 2 * (n if mod == dte.MOD_TOKEN else B * D)) * es
        log(f"variant {name}")
        out[name] = cold_and_warm(
            lambda: dte.rga_gate_add_rms_modulate_ex(x, u, g, sc, sh, 1e-6, x_out=xo, y=y,
                                                     gate_mode=mode, mod_mode=mod),
            nbytes, fused_kernel(D, dt, mode, mod))

    def fused_kernel(D, dt, mode, mod):
        # which kernel the call runs on 16-byte aligned tensors (csrc
        # gate_add_rms_modulate.hip, launch_typed)
        es = 4 if dt == "f32" else 2
        if D % 8 == 0 and D <= 8192:
            stage = (2 if mode == dte.GATE_FULL else 3) * D * es
            if mod == dte.MOD_ROW and stage <= 65536:
                return "gate_add_rms_modulate_staged_kernel"
            if mod == dte.MOD_TOKEN or dt == "f32":
                return "gate_add_rms_modulate_kernel"
        return element_fused_kernel(D, dt, mod)

    def element_fused_kernel(D, dt, mod=dte.MOD_ROW):
        # as element_norm_kernel; the fused call's LDS buffer has one more word
        if dt != "f32" and -(-(-(-D // 8)) // 64) <= 16:
            return ("gate_add_rms_modulate_regs_staged_kernel" if mod == dte.MOD_ROW
                    else "gate_add_rms_modulate_regs_kernel")
        es = 4 if dt == "f32" else 2
        if (-(-D * es // 16) + 3) * 16 <= 65536 - 256:
            return "gate_add_rms_modulate_lds_kernel"
        return "gate_add_rms_modulate_generic_kernel"

    def element_norm_kernel(norm, D, dt, mod=dte.MOD_ROW):
        # 2-byte rows of up to 16 slots of 64 groups sit in registers (two
        # rows per workgroup with row modulation); other rows up to 64 KB
        # (with two spare words, less 256 B of static LDS) are staged in LDS
        if dt != "f32" and -(-(-(-D // 8)) // 64) <= 16:
            return "modulate_regs_staged_kernel" if mod == dte.MOD_ROW else "modulate_regs_kernel"
        es = 4 if dt == "f32" else 2
        if (-(-D * es // 16) + 2) * 16 <= 65536 - 256:
            return "modulate_lds_kernel"
        return f"{norm}_modulate_generic_kernel"

    # the ideogram4 shape of the residual-gate page's table, bf16, its seeded case
    c = EXTRA_CASES["ideogram4"]
    h = make_inputs(c)
    to = lambda a: torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)
    dx, du, dg = to(h["x"]), to(h["u"]), to(h["g"])
    do = torch.empty_like(dx)
    log(f"variant {c.name}")
    out[c.name + "_gate_add"] = cold_and_warm(
        lambda: dte.rga_residual_gate_add(dx, du, dg, out=do, gate_mode=c.gate),
        (3 * c.elems + c.B * c.D) * 2, "gate_add_bcast_kernel")
    out[c.name + "_gate_add"]["shape"] = [c.B, c.L, c.D]
    del dx, du, dg, do

    # LayerNorm modulation at the modulation shape
    def ln(name, B, L, D, dt, mod):
        mshape = (B, L, D) if mod == dte.MOD_TOKEN else (B, 1, D)
        x = draw((B, L, D), dt, 2.0)
        sc, sh = draw(mshape, dt, 0.1), draw(mshape, dt, 0.1)
        o = torch.empty_like(x)
        n = B * L * D
        nbytes = (2 * n + 2 * (n if mod == dte.MOD_TOKEN else B * D)) * x.element_size()
        log(f"variant {name}")
        out[name] = cold_and_warm(
            lambda: dte.rga_ln_modulate(x, sc, sh, 1e-6, out=o, mod_mode=mod), nbytes,
            "ln_modulate_kernel" if D % 8 == 0 else element_norm_kernel("ln", D, dt, mod))

    # tanh-GELU on the FFN intermediate (video tokens x 4 hidden)
    def gelu(name, rows, F, dt, with_bias=False):
        x = draw((1, rows, F), dt, 2.0)
        b = draw((F,), dt) if with_bias else None
        o = torch.empty_like(x)
        nbytes = (2 * rows * F + (F if with_bias else 0)) * x.element_size()
        fast = (F % 8 == 0) if with_bias else True
        log(f"variant {name}")
        out[name] = cold_and_warm(lambda: dte.gelu_tanh(x, b, out=o), nbytes,
                                  ("gelu_tanh_bias_kernel" if with_bias else "gelu_tanh_flat_kernel")
                                  if fast else "gelu_tanh_generic_bias_kernel")

    # the compact set (default run)
    rms("f16_rms_modulate_[2,32640,4096]", 2, 32640, 4096, "f16", dte.MOD_ROW)
    ln("bf16_ln_modulate_[2,32640,4096]", 2, 32640, 4096, "bf16", dte.MOD_ROW)
    gelu("bf16_gelu_tanh_[1,32640,16384]", 32640, 16384, "bf16")
    if not full:
        torch.cuda.synchronize()
        return out

    gate("f16_bcast_gate_add_[1,32640,4096]", 1, 32640, 4096, "f16", dte.GATE_BCAST)
    gate("f16_full_gate_add_[1,8160,4096]", 1, 8160, 4096, "f16", dte.GATE_FULL)
    gate("f32_bcast_gate_add_[1,32640,4096]", 1, 32640, 4096, "f32", dte.GATE_BCAST)
    gate("f32_full_gate_add_[1,8160,4096]", 1, 8160, 4096, "f32", dte.GATE_FULL)
    rms("f32_rms_modulate_[2,32640,4096]", 2, 32640, 4096, "f32", dte.MOD_ROW)
    rms("bf16_rms_modulate_token_[2,32640,4096]", 2, 32640, 4096, "bf16", dte.MOD_TOKEN)
    fused("bf16_fused_token_[2,32640,4096]", 2, 32640, 4096, "bf16", dte.GATE_BCAST, dte.MOD_TOKEN)
    fused("f16_fused_[2,32640,4096]", 2, 32640, 4096, "f16", dte.GATE_BCAST, dte.MOD_ROW)
    # rows of a multiple of 8 elements that do not start on 128-byte lines
    # (4104: every row at another line position) and nine packs per lane (4608)
    gate("bf16_bcast_gate_add_[1,32640,4104]", 1, 32640, 4104, "bf16", dte.GATE_BCAST)
    rms("bf16_rms_modulate_[2,32640,4104]", 2, 32640, 4104, "bf16", dte.MOD_ROW)
    fused("bf16_fused_[2,32640,4104]", 2, 32640, 4104, "bf16", dte.GATE_BCAST, dte.MOD_ROW)
    rms("bf16_rms_modulate_[2,32640,4608]", 2, 32640, 4608, "bf16", dte.MOD_ROW)
    # element-wise paths: ragged D, an element offset, rows past the register limit
    gate("bf16_bcast_gate_add_ragged_[1,32640,4100]", 1, 32640, 4100, "bf16", dte.GATE_BCAST)
    gate("bf16_bcast_gate_add_offset1_[1,32640,4096]", 1, 32640, 4096, "bf16", dte.GATE_BCAST,
         offset=1)
    rms("bf16_rms_modulate_ragged_[2,32640,4100]", 2, 32640, 4100, "bf16", dte.MOD_ROW)
    fused("bf16_fused_ragged_[2,32640,4100]", 2, 32640, 4100, "bf16", dte.GATE_BCAST, dte.MOD_ROW)
    fused("f32_fused_ragged_[1,32640,4100]", 1, 32640, 4100, "f32", dte.GATE_BCAST, dte.MOD_ROW)
    rms("bf16_rms_modulate_wide_[1,8160,16384]", 1, 8160, 16384, "bf16", dte.MOD_ROW)
    rms("f32_rms_modulate_ragged_[1,32640,4100]", 1, 32640, 4100, "f32", dte.MOD_ROW)
    rms("bf16_rms_modulate_offset1_[2,32640,4096]", 2, 32640, 4096, "bf16", dte.MOD_ROW,
        offset=1)
    gate("f32_bcast_gate_add_offset1_[1,8160,4096]", 1, 8160, 4096, "f32", dte.GATE_BCAST,
         offset=1)
    ln("f16_ln_modulate_token_[2,32640,4096]", 2, 32640, 4096, "f16", dte.MOD_TOKEN)
    ln("bf16_ln_modulate_ragged_[2,32640,4100]", 2, 32640, 4100, "bf16", dte.MOD_ROW)
    gelu("bf16_gelu_tanh_bias_[1,32640,16384]", 32640, 16384, "bf16", with_bias=True)
    gelu("f16_gelu_tanh_[1,32640,16384]", 32640, 16384, "f16")
    gelu("f32_gelu_tanh_[1,8160,16384]", 8160, 16384, "f32")
    gelu("bf16_gelu_tanh_bias_ragged_[1,32640,16380]", 32640, 16380, "bf16", with_bias=True)
    torch.cuda.synchronize()
    return out


def _code_only(text: str) -> str:
    """C/C++ source with its comments removed and whitespace runs collapsed
    (string and character literals kept as they are): what the compiler
    sees, so an edit to comments alone keeps the digest."""
    out = []
    i, n = 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
            out.append(" ")
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return re.sub(r"\s+", " ", "".join(out)).strip()


def kernel_source_digest() -> str:
    """Digest of the library's sources as code: comments and layout do not
    count, so the committed counters stay valid across comment edits."""
    csrc = os.path.join(ROOT, "diffusion_transformer_elementwise_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if not name.endswith((".hip", ".hpp", ".cpp", ".py")):
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            data = f.read()
        if not name.endswith(".py"):
            data = _code_only(data.decode("utf-8")).encode("utf-8")
        h.update(name.encode() + b"\0" + data)
    return h.hexdigest()[:16]


def load_traffic(kernel: str):
    """HBM bytes per launch from committed counter summaries, only while the
    kernel sources are the ones the counters were taken on."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_digest") != kernel_source_digest():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def _row_ranges(B, n, parts):
    """(b, first, end) row ranges: each batch's first n rows cut into
    contiguous pieces, about `parts` in all."""
    per = max(1, -(-parts // B))
    step = -(-n // per)
    return [(b, a, min(a + step, n)) for b in range(B) for a in range(0, n, step)]


def cpu_baseline(host, fraction, min_seconds, log):
    """The oracle (the C oracle as it stands) on the first `fraction` of each
    launch's rows, same launch mix as one step, repeated until at least
    `min_seconds` have passed: once on one thread, once with every launch's
    rows cut into contiguous ranges over the host's cores (one oracle call per
    range on a thread pool; the C calls run outside the GIL). The two are
    checked bit-identical on one pass from the same inputs. `value` is the
    all-cores rate."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    from synth_inputs import CASES, GATE_BCAST, GATE_FULL

    def rows(a, c):
        n = max(1, int(round(c.L * fraction)))
        return np.ascontiguousarray(a[:, :n]), n

    c3, c4, c5 = CASES["c3"], CASES["c4"], CASES["c5"]
    h3, h4, h5 = host["c3"], host["c4"], host["c5"]
    x3, n3 = rows(h3["x"], c3); u3, _ = rows(h3["u"], c3); g3, _ = rows(h3["g"], c3)
    x4, n4 = rows(h4["x"], c4); u4, _ = rows(h4["u"], c4)
    x5, n5 = rows(h5["x"], c5); u5, _ = rows(h5["u"], c5)
    out3 = np.empty_like(x3)
    y5 = np.empty_like(x5)
    sample = (8 * c3.B * n3 * c3.D
              + 6 * c4.B * n4 * c4.D + 2 * c4.B * c4.D
              + 4 * c5.B * n5 * c5.D + 4 * c5.B * c5.D
              + 6 * c5.B * n5 * c5.D + 2 * c5.B * c5.D)

    def one_thread(x4, x5, out3, y5):
        oracle.gate_add(x3, u3, g3, GATE_FULL, out=out3)
        oracle.gate_add(x4, u4, h4["g"], GATE_BCAST, out=x4)
        oracle.rms_modulate(x5, h5["scale"], h5["shift"], c5.eps, out=y5)
        oracle.gate_add(x5, u5, h5["g"], GATE_BCAST, out=x5)

    threads = max(1, min(len(os.sched_getaffinity(0)), 16))
    pool = ThreadPoolExecutor(max_workers=threads)
    r3 = _row_ranges(c3.B, n3, threads)
    r4 = _row_ranges(c4.B, n4, threads)
    r5 = _row_ranges(c5.B, n5, threads)

    def launch(fn, ranges):
        for f in [pool.submit(fn, *r) for r in ranges]:
            f.result()

    def all_cores(x4, x5, out3, y5):
        launch(lambda b, a, e: oracle.gate_add(
            x3[b:b + 1, a:e], u3[b:b + 1, a:e], g3[b:b + 1, a:e], GATE_FULL,
            out=out3[b:b + 1, a:e]), r3)
        launch(lambda b, a, e: oracle.gate_add(
            x4[b:b + 1, a:e], u4[b:b + 1, a:e], h4["g"][b:b + 1], GATE_BCAST,
            out=x4[b:b + 1, a:e]), r4)
        launch(lambda b, a, e: oracle.rms_modulate(
            x5[b:b + 1, a:e], h5["scale"][b:b + 1], h5["shift"][b:b + 1], c5.eps,
            out=y5[b:b + 1, a:e]), r5)
        launch(lambda b, a, e: oracle.gate_add(
            x5[b:b + 1, a:e], u5[b:b + 1, a:e], h5["g"][b:b + 1], GATE_BCAST,
            out=x5[b:b + 1, a:e]), r5)

    # one pass each from the same inputs: the partitioned run must give the
    # single-threaded bits
    s_out = [x4.copy(), x5.copy(), np.empty_like(out3), np.empty_like(y5)]
    p_out = [x4.copy(), x5.copy(), np.empty_like(out3), np.empty_like(y5)]
    one_thread(*s_out)
    all_cores(*p_out)
    same = all(np.array_equal(a, b) for a, b in zip(s_out, p_out))
    del s_out, p_out
    if not same:
        pool.shutdown()
        raise RuntimeError("row-partitioned oracle differs from the single-threaded one")

    def timed(run):
        reps = 0
        t0 = time.perf_counter()
        while True:
            run(x4, x5, out3, y5)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                return reps, dt

    log(f"cpu baseline: oracle on {fraction:.2f} of every launch's rows, one thread "
        f"then {threads}, each for at least {min_seconds:.0f} s")
    reps1, dt1 = timed(one_thread)
    log(f"cpu baseline: 1 thread {sample * reps1 / 1e9:.2f} GB in {dt1:.1f} s ({reps1} passes)")
    repsn, dtn = timed(all_cores)
    pool.shutdown()
    log(f"cpu baseline: {threads} threads {sample * repsn / 1e9:.2f} GB in {dtn:.1f} s "
        f"({repsn} passes)")
    return {"value": round(sample * repsn / dtn / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{repsn} passes over the first {fraction:.2f} of the rows of each of "
                      f"the step's 4 launches ({sample * repsn} algorithmic bytes in "
                      f"{dtn:.1f} s), the C oracle called on contiguous row ranges from "
                      f"{threads} threads; bit-identical to one thread on one pass",
            "single_thread": {"value": round(sample * reps1 / dt1 / 1e9, 3), "unit": "GB/s",
                              "cores": 1,
                              "sample": f"{reps1} passes, {sample * reps1} algorithmic "
                                        f"bytes in {dt1:.1f} s"},
            "host_cpus": os.cpu_count()}


# ---------------------------------------------------------------------------
# rocprofv3 summaries (no GPU): per launch shape, from the csv files of
#   rocprofv3 --kernel-trace --stats --output-format csv -- python3 bench.py
#   rocprofv3 --pmc <counters> --output-format csv -- python3 bench.py ...

def _short_kernel(name: str) -> str:
    """Kernel name without 'void', the namespaces and the argument list."""
    n = name.replace("void ", "").replace("rga::(anonymous namespace)::", "")
    depth = 0
    for i, c in enumerate(n):
        if c == "<":
            depth += 1
        elif c == ">":
            depth -= 1
        elif c == "(" and depth == 0:
            return n[:i]
    return n


def known_launches():
    """(label, kernel, grid x in work-items, grid y, algorithmic bytes,
    elements) of the fixed-shape launches of the default bench and of
    --ablations 1. Grid sizes follow the launchers in csrc."""
    cdiv = lambda a, b: -(-a // b)
    out = []

    def bcast(label, B, L, D, es=2, kernel="gate_add_bcast_kernel<0>"):
        out.append((label, kernel, L * cdiv(D // 8, 64) * 64, B, (3 * B * L * D + B * D) * es,
                    B * L * D))

    def full(label, B, L, D, es=2, kernel="gate_add_full_kernel<0>"):
        n = B * L * D
        out.append((label, kernel, cdiv(n // 8 + (1 if n % 8 else 0), 64) * 64, 1, 4 * n * es, n))

    def mod(label, B, L, D, kernel, es=2):
        out.append((label, kernel, cdiv(L, 2) * 128, B, (2 * B * L * D + 2 * B * D) * es,
                    B * L * D))

    full("c3 full [1,8160,4096]", 1, 8160, 4096)
    bcast("c4 bcast in place [1,32640,4096]", 1, 32640, 4096)
    bcast("c5 bcast in place [2,32640,4096]", 2, 32640, 4096)
    mod("c5 rms_modulate [2,32640,4096]", 2, 32640, 4096, "rms_modulate_kernel<8, 0, 0, true>")
    out.append(("fused gate+rms [2,32640,4096]", "gate_add_rms_modulate_staged_kernel<8, false, 0, true>",
                16320 * 128, 2, (4 * 2 * 32640 * 4096 + 3 * 2 * 4096) * 2, 2 * 32640 * 4096))
    full("c1 full [1,126,2048]", 1, 126, 2048)
    mod("c1 rms_modulate [1,126,2048]", 1, 126, 2048, "rms_modulate_kernel<4, 0, 0, true>")
    for L in (512, 4096, 4608):
        bcast(f"c2 bcast [1,{L},3072]", 1, L, 3072)
    bcast("ideogram4 bcast [1,4096,4608]", 1, 4096, 4608)
    mod("f16 rms_modulate [2,32640,4096]", 2, 32640, 4096, "rms_modulate_kernel<8, 1, 0, true>")
    mod("bf16 LayerNorm modulation [2,32640,4096]", 2, 32640, 4096, "ln_modulate_kernel<8, 0, 0, true>")
    n = 32640 * 16384
    out.append(("bf16 tanh-GELU [1,32640,16384]", "gelu_tanh_flat_kernel<0>", n // 8, 1, 4 * n, n))
    e3, e4 = 8160 * 4096 * 2, 32640 * 4096 * 2
    for label, k, n16, nbytes in (
            ("mix 3R:1W [1,8160,4096]", "stream_kernel<3, true, 1>", e3 // 16, 4 * e3),
            ("mix 3R:1W [1,8160,4096], 2 words/lane", "stream_kernel<3, true, 2>", e3 // 32,
             4 * e3),
            ("mix 2R:1W in place [1,32640,4096], 2 words/lane", "stream_kernel<2, true, 2>",
             e4 // 32, 3 * e4),
            ("mix 2R:1W in place [1,32640,4096]", "stream_kernel<2, true, 1>", e4 // 16, 3 * e4),
            ("mix 2R:1W in place [2,32640,4096]", "stream_kernel<2, true, 1>", 2 * e4 // 16, 6 * e4),
            ("mix 1R:1W [2,32640,4096]", "stream_kernel<1, true, 1>", 2 * e4 // 16, 4 * e4),
            ("mix R [2,32640,4096], 1 word/lane", "stream_kernel<1, false, 1>", 2 * e4 // 16, 2 * e4),
            ("mix R [2,32640,4096], 2 words/lane", "stream_kernel<1, false, 2>", e4 // 16, 2 * e4),
            ("copy 1 GiB", "copy_kernel", FLUSH_BYTES // 16, 2 * FLUSH_BYTES),
            ("copy 1 GiB at line offset 0", "copy_kernel", line_copy_bytes(0) // 16,
             2 * line_copy_bytes(0)),
            ("copy 1 GiB at line offset 16", "copy_kernel", line_copy_bytes(16) // 16,
             2 * line_copy_bytes(16)),
            ("copy 1 GiB at line offset 64", "copy_kernel", line_copy_bytes(64) // 16,
             2 * line_copy_bytes(64)),
            ("copy 1 GiB at line offset 112", "copy_kernel", line_copy_bytes(112) // 16,
             2 * line_copy_bytes(112)),
            ("flush read 1 GiB", "read_kernel", 256 * 1024, FLUSH_BYTES)):
        out.append((label, k, n16 if k != "read_kernel" else n16, 1, nbytes, 0))
    for k, name in enumerate(SCHEDULES):
        rows = 2 * (2 if k >= 3 else 1)  # rows per workgroup
        gx = cdiv(32640, rows) * 128
        out.append((f"schedule {name}: rms_modulate [2,32640,4096]",
                    f"rms_modulate_variant_kernel<{k}>", gx, 2,
                    (2 * 2 * 32640 * 4096 + 2 * 2 * 4096) * 2, 2 * 32640 * 4096))
        out.append((f"schedule {name}: fused bcast [2,32640,4096]",
                    f"gate_add_rms_modulate_variant_kernel<{k}>", gx, 2,
                    (4 * 2 * 32640 * 4096 + 3 * 2 * 4096) * 2, 2 * 32640 * 4096))
    for T in (1, 2, 4, 8):
        for sp, pname in ((0, "nt"), (1, "plain"), (2, "device")):
            out.append((f"ablation c4 bcast, {T} rows/wave, store {pname}",
                        f"gate_add_bcast_rows_kernel<{T}, {sp}>", cdiv(32640, T) * 8 * 64, 1,
                        (3 * 32640 * 4096 + 4096) * 2, 32640 * 4096))
    return out


def _dispatch_groups(rows, grid_of):
    """{(kernel, grid_x, grid_y): [row, ...]} with kernel = short name."""
    groups = {}
    for r in rows:
        groups.setdefault((_short_kernel(r["Kernel_Name"]),) + grid_of(r), []).append(r)
    return groups


def summarize(argv):
    import csv
    what = argv[0]
    if what == "trace":
        rows = list(csv.DictReader(open(argv[1])))
        bench_line = None
        if len(argv) > 2:
            with open(argv[2]) as f:
                for line in f:
                    if line.startswith("{"):
                        bench_line = json.loads(line)
        g = _dispatch_groups(rows, lambda r: (int(r["Grid_Size_X"]), int(r["Grid_Size_Y"])))
        dur = lambda rs: [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rs]
        print("--stats view (every launch of the run; one kernel name spans several shapes)")
        by_name = {}
        for (k, gx, gy), rs in g.items():
            by_name.setdefault(k, []).extend(dur(rs))
        print(f"{'kernel':52s} {'calls':>6s} {'avg us':>9s} {'min us':>9s} {'max us':>9s}")
        for k, ds in sorted(by_name.items(), key=lambda kv: -sum(kv[1])):
            if not k.startswith(("gate_", "rms_", "ln_", "gelu_", "modulate_", "stream_",
                                 "copy_", "read_", "fill_")):
                continue
            print(f"{k[:52]:52s} {len(ds):6d} {statistics.mean(ds):9.2f} {min(ds):9.2f} "
                  f"{max(ds):9.2f}")
        print()
        print("per launch shape (device durations from the kernel trace; algorithmic bytes / "
              "average duration)")
        print(f"{'launch':44s} {'kernel':44s} {'grid':>14s} {'wg':>4s} {'vgpr*':>5s} "
              f"{'calls':>5s} {'avg us':>8s} {'GB/s':>7s} {'of 8TB/s':>8s}")
        step = {}
        for label, k, gx, gy, nbytes, _ in known_launches():
            rs = g.get((k, gx, gy))
            if not rs:
                continue
            ds = dur(rs)
            avg = statistics.mean(ds)
            gbps = nbytes / (avg * 1e-6) / 1e9
            print(f"{label[:44]:44s} {k[:44]:44s} {f'{gx}x{gy}':>14s} "
                  f"{rs[0]['Workgroup_Size_X']:>4s} {rs[0]['VGPR_Count']:>5s} {len(ds):5d} "
                  f"{avg:8.2f} {gbps:7.0f} {gbps / HBM_PEAK_GBPS:8.3f}")
            step[label] = (k, ds, nbytes)
        print("* VGPR_Count as rocprofv3 reports it")
        dom = [step[l] for l in ("c4 bcast in place [1,32640,4096]",
                                 "c5 bcast in place [2,32640,4096]") if l in step]
        if dom:
            # the bench's roofline: mean bytes per launch / mean duration per
            # launch over the step's launches of the kernel (equal counts)
            n4, n5 = len(dom[0][1]), len(dom[-1][1])
            avg = (statistics.mean(dom[0][1]) + statistics.mean(dom[-1][1])) / 2
            mb = (dom[0][2] + dom[-1][2]) / 2
            print()
            print(f"gate_add_bcast_kernel<0> over the step's shapes (c4 and c5, {n4} + {n5} "
                  f"launches): avg {avg:.2f} us per launch, {mb / (avg * 1e-6) / 1e9:.1f} GB/s, "
                  f"frac {mb / (avg * 1e-6) / 1e9 / HBM_PEAK_GBPS:.4f}")
        if bench_line:
            r = bench_line["roofline"]
            print(f"the same run's bench line: roofline.avg_launch_us {r['avg_launch_us']} "
                  f"(HIP events on the launch stream), achieved {r['achieved']} GB/s, frac "
                  f"{r['frac']}; value {bench_line['value']} GB/s, ms_per_step "
                  f"{bench_line['ms_per_step']}")
        return
    if what == "counters":
        out_json = argv[1]
        vals = {}   # (kernel, grid) -> counter -> [values]
        valu_us = {}  # (kernel, grid) -> durations of the dispatches that counted VALU
        for path in argv[2:]:
            for r in csv.DictReader(open(path)):
                key = (_short_kernel(r["Kernel_Name"]), int(r["Grid_Size"]))
                vals.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(
                    float(r["Counter_Value"]))
                if r["Counter_Name"] == "SQ_INSTS_VALU":
                    valu_us.setdefault(key, []).append(
                        (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        mean = lambda v: sum(v) / len(v)
        copy = vals.get(("copy_kernel", FLUSH_BYTES // 16), {})
        fs = ws = None
        if "FETCH_SIZE" in copy:
            fs = FLUSH_BYTES / (mean(copy["FETCH_SIZE"]) * 1024)
        if "WRITE_SIZE" in copy:
            ws = FLUSH_BYTES / (mean(copy["WRITE_SIZE"]) * 1024)
        print("calibration on the 1 GiB copy (1 GiB read, 1 GiB written): "
              f"FETCH_SIZE scale {fs if fs is None else round(fs, 5)}, "
              f"WRITE_SIZE scale {ws if ws is None else round(ws, 5)}")
        names = sorted({c for v in vals.values() for c in v})
        print(f"counters: {', '.join(names)} (mean per dispatch; instruction counts per "
              "element are wave instructions x 64 / elements)")
        hdr = f"{'launch':44s} {'n':>3s} {'read B':>12s} {'write B':>12s} {'traffic/alg':>11s}"
        extra = [c for c in names if c not in ("FETCH_SIZE", "WRITE_SIZE")]
        for c in extra:
            hdr += f" {c[:16]:>16s}"
        if "SQ_INSTS_VALU" in names:
            hdr += f" {'VALU use':>9s}"
        print(hdr)
        traffic = {}
        for label, k, gx, gy, nbytes, elems in known_launches():
            v = vals.get((k, gx * gy))
            if not v:
                continue
            rd = mean(v["FETCH_SIZE"]) * 1024 * fs if ("FETCH_SIZE" in v and fs) else None
            wr = mean(v["WRITE_SIZE"]) * 1024 * ws if ("WRITE_SIZE" in v and ws) else None
            n = max(len(x) for x in v.values())
            line = f"{label[:44]:44s} {n:3d} "
            line += f"{rd:12.0f} " if rd is not None else f"{'-':>12s} "
            line += f"{wr:12.0f} " if wr is not None else f"{'-':>12s} "
            line += f"{(rd + wr) / nbytes:11.4f}" if rd is not None and wr is not None else f"{'-':>11s}"
            for c in extra:
                if c in v and elems:
                    per = mean(v[c]) * (64 if c.startswith("SQ_INSTS") else 1) / elems
                    line += f" {per:16.4f}"
                elif c in v:
                    line += f" {mean(v[c]):16.0f}"
                else:
                    line += f" {'-':>16s}"
            if "SQ_INSTS_VALU" in names:
                d = valu_us.get((k, gx * gy))
                if d and "SQ_INSTS_VALU" in v:
                    # lane-ops over the non-packed issue rate: 256 CUs x 64 lanes x 2.4 GHz
                    use = mean(v["SQ_INSTS_VALU"]) * 64 / (mean(d) * 1e-6 * 256 * 64 * 2.4e9)
                    line += f" {use:9.3f}"
                else:
                    line += f" {'-':>9s}"
            print(line)
            if rd is not None and wr is not None:
                traffic[label] = {"kernel": k, "bytes_per_launch": round(rd + wr),
                                  "algorithmic_bytes": nbytes}
        if out_json and traffic:
            step = {}
            for label, kk in (("c3 full [1,8160,4096]", "gate_add_full_kernel"),
                              ("c5 rms_modulate [2,32640,4096]", "rms_modulate_kernel"),
                              ("fused gate+rms [2,32640,4096]",
                               "gate_add_rms_modulate_staged_kernel")):
                if label in traffic:
                    step[kk] = {"bytes_per_launch": traffic[label]["bytes_per_launch"],
                                "launches_averaged": 1}
            b = [traffic[l]["bytes_per_launch"] for l in ("c4 bcast in place [1,32640,4096]",
                                                          "c5 bcast in place [2,32640,4096]")
                 if l in traffic]
            if len(b) == 2:
                step["gate_add_bcast_kernel"] = {"bytes_per_launch": round(sum(b) / 2),
                                                 "launches_averaged": 2}
            with open(out_json, "w") as f:
                json.dump({"source_digest": kernel_source_digest(),
                           "about": "HBM bytes per launch (FETCH_SIZE and WRITE_SIZE, scaled by "
                                    "the copy-kernel calibration) for the bench's launches; used "
                                    "only while the kernel sources match the digest",
                           "calibration": {"fetch_scale": fs, "write_scale": ws},
                           "kernels": step, "launches": traffic}, f, indent=1)
                f.write("\n")
        return
    if what == "variants":
        summarize_variants(argv[1], argv[2:])
        return
    raise SystemExit(f"--summarize: unknown kind {what!r}")


def _library_dispatches(paths):
    """[(dispatch id, short kernel name, grid work-items, {column: value}),
    ...] in dispatch order for the library's compute kernels (the cache
    flush excluded), from kernel-trace or counter csv files; a counter file
    has one row per counter per dispatch, merged here."""
    import csv
    by_id = {}
    for path in paths:
        for r in csv.DictReader(open(path)):
            if "rga::" not in r["Kernel_Name"]:
                continue
            k = _short_kernel(r["Kernel_Name"])
            if k == "read_kernel":
                continue
            if "Grid_Size" in r:
                grid = int(r["Grid_Size"])
            else:
                grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            d = by_id.setdefault(int(r["Dispatch_Id"]), (k, grid, {}))[2]
            d["us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            d["vgpr"] = r.get("VGPR_Count")
            if "Counter_Name" in r:
                d[r["Counter_Name"]] = float(r["Counter_Value"])
    return [(i,) + by_id[i] for i in sorted(by_id)]


def summarize_variants(bench_json, paths):
    """Per-variant kernel, grid and device time (kernel trace) or HBM bytes
    and instruction counts (counter csv files) for a run with
    '--variants 1 --fused-reps 0 --ablations 0', where the variants' calls
    are the run's last library dispatches: each variant is cold_reps calls
    after a flush, then 100 back to back, all one kernel and grid. Matching
    runs backwards from the last dispatch and checks that every call of a
    variant is the same launch of the kernel the bench names."""
    line = None
    with open(bench_json) as f:
        for s in f:
            if s.startswith("{"):
                line = json.loads(s)
    variants = line["variants"]
    disp = _library_dispatches(paths)
    counters = sorted({c for _, _, _, d in disp for c in d if c.isupper()})
    calib = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        cp = [d[c] for _, k, g, d in disp if k == "copy_kernel" and g == FLUSH_BYTES // 16
              and c in d]
        if cp:
            calib[c] = FLUSH_BYTES / (sum(cp) / len(cp) * 1024)
    if calib:
        print("calibration on the 1 GiB copy: " + ", ".join(
            f"{c} scale {v:.5f}" for c, v in calib.items()))
    rows = []
    end = len(disp)
    for name in reversed(list(variants)):
        v = variants[name]
        n = v["cold_reps"] + v["warm_reps"]
        k, g = disp[end - 1][1], disp[end - 1][2]
        start = end - n
        if start < 0 or any((x[1], x[2]) != (k, g) for x in disp[start:end]):
            raise SystemExit(f"variants: dispatches before the end do not match {name}")
        if not k.startswith(v["kernel"]):
            raise SystemExit(f"variants: {name} ran {k}, the bench names {v['kernel']}")
        rows.append((name, v, k, g, [x[3] for x in disp[start:end]]))
        end = start
    rows.reverse()
    mean = lambda a: sum(a) / len(a)

    def elements(name, v):
        m = re.search(r"\[([\d,]+)\]", name)
        s = v.get("shape") or ([int(t) for t in m.group(1).split(",")] if m else None)
        return s[0] * s[1] * s[2] if s else None
    if "FETCH_SIZE" in counters or "WRITE_SIZE" in counters:
        hdr = f"{'variant':44s} {'kernel':46s} {'read B':>11s} {'write B':>11s} {'traffic/alg':>11s}"
        for c in counters:
            if c.startswith("SQ_"):
                hdr += f" {c[3:17]:>14s}"
        print(hdr)
        print("(SQ_ columns: wave instructions x 64 per element)")
        for name, v, k, g, ds in rows:
            elems = elements(name, v)
            out = f"{name[:44]:44s} {k[:46]:46s}"
            tot = 0
            for c in ("FETCH_SIZE", "WRITE_SIZE"):
                vals = [d[c] for d in ds if c in d]
                if vals and c in calib:
                    b = mean(vals) * 1024 * calib[c]
                    tot += b
                    out += f" {b:11.0f}"
                else:
                    tot = None if vals else tot
                    out += f" {'-':>11s}"
            have = all(any(c in d for d in ds) for c in ("FETCH_SIZE", "WRITE_SIZE"))
            out += f" {tot / v['bytes']:11.4f}" if have and tot else f" {'-':>11s}"
            for c in counters:
                if c.startswith("SQ_"):
                    vals = [d[c] for d in ds if c in d]
                    out += f" {mean(vals) * 64 / elems:14.4f}" if vals and elems else f" {'-':>14s}"
            print(out)
        return
    print(f"{'variant':44s} {'kernel':50s} {'grid':>9s} {'vgpr*':>5s} {'cold us':>8s} "
          f"{'b2b us':>8s} {'trace cold':>10s} {'trace b2b':>9s} {'of 8TB/s':>8s}")
    for name, v, k, g, ds in rows:
        nc = v["cold_reps"]
        tc = statistics.median([d["us"] for d in ds[:nc]]) if nc > 0 else float("nan")
        tw = mean([d["us"] for d in ds[nc:]])
        print(f"{name[:44]:44s} {k[:50]:50s} {g:9d} {str(ds[0]['vgpr']):>5s} "
              f"{v['cold_us_median']:8.2f} {v['back_to_back_us']:8.2f} {tc:10.2f} {tw:9.2f} "
              f"{v['frac_of_hbm_peak']:8.4f}")
    print("cold us, b2b us: the bench's HIP events (cold = median after a 1 GiB flush; b2b = mean "
          "of 100 consecutive calls); trace cold / b2b: the same calls' device durations from the "
          "kernel trace (median / mean); of 8TB/s: algorithmic bytes / cold median; "
          "* VGPR_Count as rocprofv3 reports it")


if __name__ == "__main__":
    main()
