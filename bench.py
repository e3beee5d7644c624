#!/usr/bin/env python3
"""Benchmark of the MoE EP low-latency dispatch + combine path on one MI355X.

One step = layout -> dispatch -> combine (ep_layout_dispatch, one launch for
small batches, then ep_combine) over one batch of seeded synthetic inputs
already resident in HBM (the expert computation between
dispatch and combine is outside the path; combine reads synthetic expert
outputs).  Default workload: 128 tokens x hidden 7168, top-8 of 288 experts
in 16 destination partitions, fp8 e4m3fn dispatch with per-128 scales, bf16
combine -- the low-latency test shape the sources quote (MoRI PR #614,
test_low_latency.py argument paragraph).  Steps are replayed from a HIP
graph (small-token regime) and timed with HIP events on the stream they run
on, between a synchronize on both sides.

Prints ONE JSON line: value = algorithmic HBM bytes per step / time per
step (GB/s; metadata excluded), plus the roofline of the dominant kernel and
the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dispatch+combine µs and HBM GB/s (% of 8 TB/s) at 128 tok×7168, topk 8"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published


def algo_bytes(wl, N):
    """Bytes the method must move (payload only): per phase and per step."""
    T, H = wl.T, wl.H
    if wl.payload == "fp8":
        disp = T * 2 * H + N * (H + (H // 128) * 4)
    else:
        disp = T * 2 * H + N * 2 * H
    comb = N * 2 * H + T * 2 * H
    return {"dispatch": disp, "combine": comb, "layout": 0, "step": disp + comb}


class Path:
    """Device inputs + persistent buffers for one workload."""

    def __init__(self, wl, seed=None):
        import torch
        import combine_ep_layout_05_amd as ep
        from workloads import generate
        self.ep, self.torch, self.wl = ep, torch, wl
        self.d = generate(wl, seed=seed)
        dev = torch.device("cuda:0")

        def up(a, dt=None):
            t = torch.from_numpy(np.ascontiguousarray(a))
            return (t.view(dt) if dt is not None else t).to(dev)
        self.idx = up(self.d["idx"])
        self.w = up(self.d["w"])
        self.x = up(self.d["x"].view(np.int16), torch.bfloat16)
        self.y = up(self.d["y"].view(np.int16), torch.bfloat16)
        self.buf = ep.EpBuffers(wl.T, wl.H, wl.K, wl.E, wl.P, payload=wl.payload,
                                geometry=GEOMETRY)
        self.stream = torch.cuda.Stream()
        self.N = self.d["N"]

    def enqueue(self, phase="step"):
        """step: ep_layout_dispatch (one launch for small batches) + ep_combine;
        step3: ep_layout + ep_dispatch + ep_combine; or a single phase."""
        s, b = self.stream, self.buf
        if phase in ("step", "layout_dispatch"):
            b.layout_dispatch(self.idx, self.x, s)
        if phase in ("step3", "layout"):
            b.layout(self.idx, s)
        if phase in ("step3", "dispatch"):
            b.dispatch(self.x, s)
        if phase in ("step", "step3", "combine"):
            b.combine(self.y, self.w, s)

    def capture(self, phase="step", reps=1):
        ep, torch = self.ep, self.torch
        with torch.cuda.stream(self.stream):
            ep.ep_graph_begin(self.stream)
            for _ in range(reps):
                self.enqueue(phase)
            return ep.ep_graph_end(self.stream)

    def time_graph(self, g, launches, warmup=3):
        torch = self.torch
        for _ in range(warmup):
            g.launch(self.stream)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for _ in range(launches):
            g.launch(self.stream)
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / launches      # us per launch

    def time_eager_bound(self, iters, warmup=3):
        """Eager steps through a BoundStep (arguments marshalled once)."""
        torch = self.torch
        bs = self.ep.BoundStep(self.buf, self.idx, self.x, self.y, self.w, self.stream)
        for _ in range(warmup):
            bs.step()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for _ in range(iters):
            bs.step()
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / iters

    def time_eager(self, iters, warmup=3, phase="step"):
        torch = self.torch
        for _ in range(warmup):
            self.enqueue(phase)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for _ in range(iters):
            self.enqueue(phase)
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / iters

    def phase_us(self, phase, reps=50, launches=10):
        """Average duration of one launch of a phase: a graph of `reps`
        back-to-back launches, replayed `launches` times, timed with events."""
        g = self.capture(phase, reps)
        us = self.time_graph(g, launches) / reps
        g.destroy()
        return us


class DedupPath(Path):
    """The per-destination (dedup) step on the same inputs: ep_layout (expert
    rows for the expert outputs) + ep_dedup_layout + the dedup dispatch
    (ep_dispatch with K = P over tp_row) + ep_combine_partial +
    ep_combine_reduce."""

    def __init__(self, wl, seed=None):
        super().__init__(wl, seed)
        self.db = self.ep.EpDedupBuffers(wl.T, wl.H, wl.K, wl.E, wl.P, payload=wl.payload)
        self.enqueue("dedup_layout")
        self.torch.cuda.synchronize()
        self.M = int(self.db.part_token_offset[wl.P].item())

    def enqueue(self, phase="dedup"):
        """dedup_step: ep_dedup_layout_dispatch (one launch for small batches)
        + ep_combine_partial + ep_combine_reduce; dedup: the same step with
        ep_layout, ep_dedup_layout and ep_dispatch as separate calls."""
        s, b, db = self.stream, self.buf, self.db
        if phase in ("dedup_step", "dedup_layout_dispatch"):
            db.layout_dispatch(self.idx, self.x, b, s)
        if phase in ("dedup_step", "combine_partial", "combine_reduce"):
            if phase != "combine_reduce":
                db.combine_partial(self.y, b.row_of_pair, self.w, s)
            if phase != "combine_partial":
                db.combine_reduce(s)
            return
        if phase in ("dedup", "layout"):
            b.layout(self.idx, s)
        if phase in ("dedup", "dedup_layout"):
            db.layout(self.idx, s)
        if phase in ("dedup", "dedup_dispatch"):
            db.dispatch(self.x, s)
        if phase == "dedup":
            db.combine_partial(self.y, b.row_of_pair, self.w, s)
            db.combine_reduce(s)


def dedup_bytes(wl, N, M):
    """Algorithmic HBM bytes of the dedup step's kernels, and the bytes that
    would cross between GPUs (rows sent to a destination and back)."""
    T, H = wl.T, wl.H
    row = H + (H // 128) * 4 if wl.payload == "fp8" else 2 * H
    b = {"dedup_dispatch": T * 2 * H + M * row,
         "dedup_layout_dispatch": T * 2 * H + M * row,
         "combine_partial": N * 2 * H + M * 2 * H,
         "combine_reduce": M * 2 * H + T * 2 * H}
    b["link_dedup"] = M * row + M * 2 * H
    b["link_plain"] = N * row + N * 2 * H
    return b


def dedup_report(wl, steps=1000):
    p = DedupPath(wl)
    b = dedup_bytes(wl, p.N, p.M)
    us = time_steps(p, steps, 20, "graph", "dedup_step")
    us_sep = time_steps(p, steps, 20, "graph", "dedup")
    ph = {k: p.phase_us(k) for k in ("dedup_layout_dispatch", "layout", "dedup_layout",
                                     "dedup_dispatch", "combine_partial", "combine_reduce")}
    out = {"workload": wl.name, "E": wl.E, "P": wl.P, "pairs_N": p.N, "copies_M": p.M,
           "us_per_step_graph": round(us, 3),
           "step": "ep_dedup_layout_dispatch + ep_combine_partial + ep_combine_reduce",
           "us_per_step_graph_separate_calls": round(us_sep, 3),
           "phases_us": {k: round(v, 3) for k, v in ph.items()},
           "phase_GBps": {k: round(b[k] / (ph[k] * 1e-6) / 1e9, 1)
                          for k in ("dedup_layout_dispatch", "dedup_dispatch", "combine_partial",
                                    "combine_reduce")},
           "link_bytes_dedup": b["link_dedup"], "link_bytes_plain": b["link_plain"],
           "link_bytes_ratio": round(b["link_dedup"] / max(b["link_plain"], 1), 4)}
    del p
    return out


def recorded_traffic(phase, workload):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    readings (profiles/traffic.txt), or None when there is no reading for this
    kernel and workload or the kernel's sources changed since it was taken."""
    from combine_ep_layout_05_amd import build as B
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        f = line.split()
        kv = dict(x.split("=", 1) for x in f[2:])
        if f[0] == phase and f[1] == workload:
            if kv.get("source_digest") != B.source_digest(phase):
                return None
            return int(float(kv["traffic_bytes"]))
    return None


def cpu_baseline(wl, d, N, min_seconds):
    """The oracle as it stands (single-threaded C), full steps of the same
    workload on the host, repeated until min_seconds have elapsed."""
    import oracle
    bytes_step = algo_bytes(wl, N)["step"]
    n, t0 = 0, time.perf_counter()
    while True:
        lo = oracle.layout(d["idx"], wl.E, wl.P)
        if wl.payload == "fp8":
            oracle.dispatch_fp8(d["x"], lo["row_of_pair"], wl.K)
        else:
            oracle.dispatch_bf16(d["x"], lo["row_of_pair"], wl.K)
        oracle.combine(d["y"], lo["row_of_pair"], d["w"], wl.T, wl.H, wl.K)
        n += 1
        el = time.perf_counter() - t0
        if el >= min_seconds and n >= 2:
            break
    per = el / n
    return {"value": round(bytes_step / per / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "%d full steps (layout+dispatch+combine) of %s, %.1f ms/step" % (n, wl.name, per * 1e3)}


STEPS_PER_GRAPH = 50
GEOMETRY = "tuned"      # launch geometry of dispatch/combine: the saved tuner rules for the shape


def time_steps(p, steps, warmup, mode, phase="step"):
    """us per step.  mode "graph": graphs of STEPS_PER_GRAPH whole steps
    (device time per step; one graph launch per STEPS_PER_GRAPH steps);
    "graph1": one graph launch per step (adds the host's graph-launch cost);
    "eager": every call enqueued from the host."""
    torch = p.torch
    if mode == "eager":
        return p.time_eager(steps, warmup, phase)
    per = min(STEPS_PER_GRAPH, steps) if mode == "graph" else 1
    g = p.capture(phase, per)
    launches = max(1, steps // per)
    for _ in range(max(1, warmup // per)):
        g.launch(p.stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(p.stream)
    for _ in range(launches):
        g.launch(p.stream)
    e1.record(p.stream)
    torch.cuda.synchronize()
    g.destroy()
    return e0.elapsed_time(e1) * 1e3 / (launches * per)


def single_step_us(p, reps, flush_bytes=0):
    """Median device time of one step (a BoundStep's two launches between two
    events), each step preceded -- outside the events -- by a write of
    flush_bytes that evicts the step's data from L2 and the memory-side cache
    (cold), or by nothing (warm); then a bounded GPU spin keeps the GPU busy
    while the host enqueues the events and the step, so no host time is inside
    the events."""
    torch = p.torch
    bs = p.ep.BoundStep(p.buf, p.idx, p.x, p.y, p.w, p.stream)
    flush = torch.empty(max(flush_bytes, 1), dtype=torch.uint8, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for i in range(reps + 2):
        with torch.cuda.stream(p.stream):
            if flush_bytes:
                flush.fill_(i & 0xFF)
            torch.cuda._sleep(200000)       # bounded spin: the GPU stays busy while the host enqueues
        e0.record(p.stream)
        bs.step()
        e1.record(p.stream)
        torch.cuda.synchronize()
        if i >= 2:
            times.append(e0.elapsed_time(e1) * 1e3)
    del flush
    return float(np.median(times))


def native_loop(wl, steps=5000):
    """ep_layout_dispatch + ep_combine enqueued back to back from C++ (the
    package's ep_loop program, a child process started before this process
    touches the GPU): host and wall microseconds per step, i.e. what a native
    serving loop pays without an interpreter or graph launches in between.
    Uses the library's default launch geometry."""
    exe = os.path.join(ROOT, "combine_ep_layout_05_amd", "ep_loop")
    if not os.path.exists(exe):
        return None
    r = subprocess.run([exe, str(wl.T), str(wl.H), str(wl.K), str(wl.E), str(wl.P), wl.payload,
                        str(steps)], capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        return {"error": (r.stderr or r.stdout)[-300:]}
    return json.loads(r.stdout.strip().splitlines()[-1])


def measure(wl, steps, warmup, mode="graph", phase="step"):
    p = Path(wl)
    b = algo_bytes(wl, p.N)
    return p, b, time_steps(p, steps, warmup, mode, phase)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="ll_128x7168")
    ap.add_argument("--eager", action="store_true", help="time host-launched steps, no graph")
    ap.add_argument("--unfused", action="store_true",
                    help="step = ep_layout + ep_dispatch + ep_combine (default: ep_layout_dispatch + ep_combine)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--default-geometry", action="store_true",
                    help="launch dispatch/combine with the library's default geometry, not the tuned rules")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-targets", action="store_true")
    ap.add_argument("--no-dedup", action="store_true")
    ap.add_argument("--only", choices=["layout", "dispatch", "combine", "layout_dispatch", "step",
                                       "step3", "dedup_layout", "dedup_dispatch", "combine_partial",
                                       "combine_reduce", "dedup", "dedup_layout_dispatch",
                                       "dedup_step"],
                    help="profiling mode: launch only this phase (eagerly) steps times, print nothing else")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="profiling mode: first run one device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the EP traffic and runs on one GPU only; "
              "the multi-GPU exchange is not implemented (asked for --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    from workloads import WORKLOADS
    wl = WORKLOADS[args.workload]
    global GEOMETRY
    if args.default_geometry:
        GEOMETRY = None

    if args.only or args.calib_copy_mib:
        if args.calib_copy_mib:
            n = args.calib_copy_mib << 20
            src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
            dst = torch.empty_like(src)
            torch.cuda.synchronize()
            dst.copy_(src)
            torch.cuda.synchronize()
            print("calib copy %d bytes" % n, flush=True)
        if args.only:
            p = DedupPath(wl) if args.only.startswith(("dedup", "combine_")) else Path(wl)
            p.enqueue("dedup" if isinstance(p, DedupPath) else "step3")
            torch.cuda.synchronize()
            for _ in range(args.warmup + args.steps):
                p.enqueue(args.only)
            torch.cuda.synchronize()
            print("profiled %s x%d on %s" % (args.only, args.warmup + args.steps, wl.name), flush=True)
        return

    native = None
    if not args.no_targets:      # before this process initialises the GPU
        native = {w.name: native_loop(w) for w in (wl, WORKLOADS["sweep_4x6144"])}

    step = "step3" if args.unfused else "step"
    mode = "eager" if args.eager else "graph"
    p, b, us = measure(wl, args.steps, args.warmup, mode=mode, phase=step)
    eager_us = time_steps(p, 500, 20, "eager", step)
    eager_bound_us = p.time_eager_bound(500, 20) if step == "step" else None
    graph1_us = time_steps(p, 1000, 20, "graph1", step)
    warm1_us = single_step_us(p, 50, 0)
    cold1_us = single_step_us(p, 50, 512 << 20)
    phases = {ph: p.phase_us(ph) for ph in ("layout_dispatch", "layout", "dispatch", "combine")}
    b["layout_dispatch"] = b["dispatch"]
    cand = ("dispatch", "combine") if args.unfused else ("layout_dispatch", "combine")
    dom = max(cand, key=lambda ph: phases[ph])
    achieved = b[dom] / (phases[dom] * 1e-6) / 1e9
    roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(dom, wl.name),
            "bytes_per_launch": b[dom], "us_per_launch": round(phases[dom], 3)}
    value = b["step"] / (us * 1e-6) / 1e9

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6),
        "us_per_step": round(us, 3),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "payload": "fp8_e4m3fn+fp32 per-128 scales dispatch, bf16 combine" if wl.payload == "fp8"
        else "bf16 dispatch, bf16 combine",
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens": wl.T, "hidden": wl.H, "experts": wl.E,
                   "partitions": wl.P, "topk": wl.K, "valid_pairs": p.N,
                   "timing": "eager host launches" if args.eager else
                   "HIP graphs of %d whole steps, replayed" % STEPS_PER_GRAPH,
                   "step": "ep_layout + ep_dispatch + ep_combine" if args.unfused
                   else "ep_layout_dispatch + ep_combine",
                   "parallelism": "single GPU (partitions stand in for EP ranks)",
                   "geometry": {k: list(v) for k, v in p.buf.geometry.items()} or "library default"},
        "bytes_per_step": b["step"],
        "phases_us": {k: round(v, 3) for k, v in phases.items()},
        "eager_us_per_step": round(eager_us, 3),
        "eager_bound_us_per_step": None if eager_bound_us is None else round(eager_bound_us, 3),
        "graph1_us_per_step": round(graph1_us, 3),
        "single_step_us": {"warm": round(warm1_us, 3), "cold_after_512MB_write": round(cold1_us, 3)},
        "roofline": roof,
    }

    if not args.no_targets:
        tg = {"native_loop_us_per_step": native}
        pw, bw_, us4 = measure(WORKLOADS["sweep_4x6144"], 2000, 50)
        tg["sweep_4x6144_us_per_step_graph"] = round(us4, 3)
        tg["sweep_4x6144_us_per_step_graph1"] = round(time_steps(pw, 1000, 20, "graph1"), 3)
        tg["sweep_4x6144_us_per_step_eager"] = round(time_steps(pw, 500, 20, "eager"), 3)
        tg["sweep_4x6144_us_per_step_eager_bound"] = round(pw.time_eager_bound(500, 20), 3)
        tg["sweep_4x6144_target_us"] = 15.0
        for tt in (8, 16):
            tg["sweep_%dx6144_us_per_step_graph" % tt] = round(
                measure(WORKLOADS["sweep_%dx6144" % tt], 2000, 50)[2], 3)
        del pw
        pb, bb, usb = measure(WORKLOADS["bw_4096x7168_zipf"], 100, 10)
        tg["bw_4096x7168_zipf_us_per_step"] = round(usb, 2)
        tg["bw_4096x7168_zipf_hbm_frac"] = round(bb["step"] / (usb * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        tg["bw_4096x7168_zipf_target_frac"] = 0.60
        tg["bw_4096x7168_zipf_phases_us"] = {ph: round(pb.phase_us(ph, reps=10, launches=3), 2)
                                            for ph in ("layout", "dispatch", "combine")}
        tg["sweep_4x6144_unfused_us_per_step_graph"] = round(
            measure(WORKLOADS["sweep_4x6144"], 2000, 50, phase="step3")[2], 3)
        pm, bm, usm = measure(WORKLOADS["masked_16384x4096_bf16"], 20, 2)
        tg["masked_16384x4096_bf16_us_per_step"] = round(usm, 2)
        tg["masked_16384x4096_bf16_hbm_frac"] = round(bm["step"] / (usm * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        del pm
        del pb
        res["targets"] = tg

    if not args.no_dedup:
        res["dedup"] = [dedup_report(wl),
                        dedup_report(wl.with_(name=wl.name + "_e32p8", E=32, P=8))]

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, p.d, p.N, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
