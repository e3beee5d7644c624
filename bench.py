#!/usr/bin/env python3
"""Benchmark of the MoE EP low-latency dispatch + combine path on one MI355X.

One step = layout -> dispatch -> combine (ep_layout_dispatch, one launch for
small batches, then ep_combine) over one batch of seeded synthetic inputs
already resident in HBM (the expert computation between dispatch and combine
is outside the path; combine reads synthetic expert outputs).  Default
workload: 128 tokens x hidden 7168, top-8 of 288 experts in 16 destination
partitions, fp8 e4m3fn dispatch with per-128 scales, bf16 combine -- the
low-latency test shape the sources quote (MoRI PR #614, test_low_latency.py
argument paragraph).

Timing.  Steps are recorded into HIP graphs and timed with HIP events on the
stream they run on, between a synchronize on both sides; a bounded GPU spin
ahead of the first event keeps the host's graph-launch time out of the timed
region.  The headline times samples of exactly --steps whole steps, enough
samples for at least 1000 timed steps, and reports the median sample.

Prints ONE JSON line: value = algorithmic bytes per step / time per step
(GB/s; metadata excluded) with the 26 MB working set cache-warm (it stays in
L2 and the 256 MB memory-side cache from one step to the next, as in a
serving loop that reuses its buffers), and beside it the same step over 16
rotating input/output sets (415 MB, nothing left in the caches: the HBM
figure); the roofline of the dominant kernel in both states; the other
workloads' targets; and the CPU oracle timed on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dispatch+combine µs and HBM GB/s (% of 8 TB/s) at 128 tok×7168, topk 8"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
SPIN_CYCLES = 200000           # GPU spin ahead of a timed region (about 80 us)
MIN_TIMED_STEPS = 1000         # headline: at least this many steps per sample
HEADLINE_SAMPLES = 7
STREAM_SETS = 16               # rotating sets for the HBM-streamed figure (16 x 26 MB at 128 x 7168)
GEOMETRY = "tuned"             # launch geometry: the saved tuner rules for the shape


def algo_bytes(wl, N):
    """Bytes the method must move (payload only): per phase and per step."""
    T, H = wl.T, wl.H
    if wl.payload == "fp8":
        disp = T * 2 * H + N * (H + (H // 128) * 4)
    else:
        disp = T * 2 * H + N * 2 * H
    comb = N * 2 * H + T * 2 * H
    return {"dispatch": disp, "layout_dispatch": disp, "combine": comb, "layout": 0,
            "step": disp + comb, "step3": disp + comb}


def stats(v):
    v = sorted(v)
    return {"mean": round(float(np.mean(v)), 3), "median": round(float(np.median(v)), 3),
            "min": round(float(v[0]), 3), "samples": len(v)}


class Path:
    """Device inputs + persistent buffers for one workload; `sets` copies of
    every input and output buffer (same values, different addresses) for
    steps that rotate over them."""

    def __init__(self, wl, seed=None, sets=1):
        import torch
        import combine_ep_layout_05_amd as ep
        from workloads import generate
        self.ep, self.torch, self.wl = ep, torch, wl
        self.d = generate(wl, seed=seed)
        dev = torch.device("cuda:0")

        def up(a, dt=None):
            t = torch.from_numpy(np.ascontiguousarray(a))
            return (t.view(dt) if dt is not None else t).to(dev)
        base = dict(idx=up(self.d["idx"]), w=up(self.d["w"]),
                    x=up(self.d["x"].view(np.int16), torch.bfloat16),
                    y=up(self.d["y"].view(np.int16), torch.bfloat16))
        self.sets = []
        for i in range(sets):
            s = dict(base) if i == 0 else {k: v.clone() for k, v in base.items()}
            s["buf"] = ep.EpBuffers(wl.T, wl.H, wl.K, wl.E, wl.P, payload=wl.payload,
                                    geometry=GEOMETRY)
            self.sets.append(s)
        s0 = self.sets[0]
        self.idx, self.w, self.x, self.y, self.buf = s0["idx"], s0["w"], s0["x"], s0["y"], s0["buf"]
        self.stream = torch.cuda.Stream()
        self.N = self.d["N"]

    def enqueue(self, phase="step", i=0):
        """step: ep_layout_dispatch (one launch for small batches) + ep_combine;
        step3: ep_layout + ep_dispatch + ep_combine; or a single phase; on set i."""
        st, s = self.stream, self.sets[i % len(self.sets)]
        b = s["buf"]
        if phase in ("step", "layout_dispatch"):
            b.layout_dispatch(s["idx"], s["x"], st)
        if phase in ("step3", "layout"):
            b.layout(s["idx"], st)
        if phase in ("step3", "dispatch"):
            b.dispatch(s["x"], st)
        if phase in ("step", "step3", "combine"):
            b.combine(s["y"], s["w"], st)

    def capture(self, phase="step", reps=1, rotate=False):
        ep, torch = self.ep, self.torch
        with torch.cuda.stream(self.stream):
            ep.ep_graph_begin(self.stream)
            for r in range(reps):
                self.enqueue(phase, r if rotate else 0)
            return ep.ep_graph_end(self.stream)

    def spin(self):
        with self.torch.cuda.stream(self.stream):
            self.torch.cuda._sleep(SPIN_CYCLES)

    def timed(self, graphs, steps, samples, warmup_launches=1, spin=True):
        """us per step of each sample; a sample launches `graphs` (a list of
        graph handles holding `steps` steps in all) between two events."""
        torch = self.torch
        for _ in range(warmup_launches):
            for g in graphs:
                g.launch(self.stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        out = []
        for _ in range(samples):
            if spin:
                self.spin()
            e0.record(self.stream)
            for g in graphs:
                g.launch(self.stream)
            e1.record(self.stream)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) * 1e3 / steps)
        return out

    def phase_samples(self, phase, reps=50, samples=20, rotate=False):
        """Per-launch times of one phase: a graph of `reps` back-to-back
        launches, replayed `samples` times."""
        g = self.capture(phase, reps, rotate)
        v = self.timed([g], reps, samples)
        g.destroy()
        return v

    def eager(self, iters, warmup=3, phase="step", bound=False):
        """Every call enqueued from the host (through a BoundStep when bound:
        arguments marshalled once)."""
        torch = self.torch
        if bound:
            bs = self.ep.BoundStep(self.buf, self.idx, self.x, self.y, self.w, self.stream)
            fn = bs.step
        else:
            def fn():
                self.enqueue(phase)
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for _ in range(iters):
            fn()
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / iters

    def graph1(self, launches=1000, phase="step"):
        """One-step graph replayed `launches` times between two events, the
        host's graph-launch cost included (what a serving loop that replays a
        graph per step sees; the graph is bound to the stream once)."""
        torch = self.torch
        g = self.capture(phase, 1)
        replay = g.bind(self.stream)
        for _ in range(20):
            replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for _ in range(launches):
            replay()
        e1.record(self.stream)
        torch.cuda.synchronize()
        g.destroy()
        return e0.elapsed_time(e1) * 1e3 / launches


def headline(p, steps, warmup, phase="step"):
    """The headline: HEADLINE_SAMPLES samples, each at least MIN_TIMED_STEPS
    whole steps (and at least `steps`) in HIP graphs of 50 steps launched back
    to back between two HIP events behind a GPU spin, whatever `steps` is;
    the median sample.  Beside it, samples of exactly `steps` steps (one graph
    of `steps` steps; 50-step graphs and a remainder above 100), enough for
    MIN_TIMED_STEPS steps in all: each of those pays one graph's start on the
    device, spread over `steps` steps."""
    per_sample = 50 * math.ceil(max(MIN_TIMED_STEPS, steps) / 50)
    g50 = p.capture(phase, 50)
    graphs = [g50] * (per_sample // 50)
    v = p.timed(graphs, per_sample, HEADLINE_SAMPLES,
                warmup_launches=max(1, math.ceil(warmup / per_sample)))
    desc = ("each sample: %d whole steps in HIP graphs of 50 steps launched back to back "
            "between two HIP events behind a GPU spin; %d samples (%d steps timed); value from "
            "the median sample" % (per_sample, HEADLINE_SAMPLES, per_sample * HEADLINE_SAMPLES))
    if steps <= 100:
        kg = [p.capture(phase, steps)]
    else:
        kg = [g50] * (steps // 50)
        if steps % 50:
            kg.append(p.capture(phase, steps % 50))
    samples = max(3, math.ceil(MIN_TIMED_STEPS / steps))
    vk = p.timed(kg, steps, samples, warmup_launches=1)
    desc_k = ("each sample: exactly %d whole steps (%s) between two HIP events behind a GPU "
              "spin; %d samples" % (
                  steps, "one HIP graph of %d steps" % steps if steps <= 100 else
                  "HIP graphs of 50 steps%s" % (" + one of %d" % (steps % 50) if steps % 50 else ""),
                  samples))
    for g in set(graphs + kg):
        g.destroy()
    return v, desc, vk, desc_k


def streamed(wl, phases=("layout_dispatch", "combine"), steps_per_graph=48, samples=21):
    """The step over STREAM_SETS rotating input/output sets: every step finds
    its data last touched STREAM_SETS - 1 steps earlier, evicted from L2 and
    the memory-side cache."""
    p = Path(wl, sets=STREAM_SETS)
    g = p.capture("step", steps_per_graph, rotate=True)
    v = p.timed([g], steps_per_graph, samples)
    g.destroy()
    ph = {k: float(np.median(p.phase_samples(k, reps=steps_per_graph, samples=10, rotate=True)))
          for k in phases}
    set_bytes = sum(t.numel() * t.element_size() for s in p.sets[:1] for t in
                    (s["idx"], s["w"], s["x"], s["y"], s["buf"].recv_x, s["buf"].out) +
                    ((s["buf"].recv_scales,) if s["buf"].recv_scales is not None else ()))
    del p
    return v, ph, set_bytes * STREAM_SETS


class DedupPath(Path):
    """The per-destination (dedup) step on the same inputs."""

    def __init__(self, wl, seed=None):
        super().__init__(wl, seed)
        self.db = self.ep.EpDedupBuffers(wl.T, wl.H, wl.K, wl.E, wl.P, payload=wl.payload,
                                         geometry="tuned" if GEOMETRY else None)
        self.enqueue("dedup_layout")
        self.torch.cuda.synchronize()
        self.M = int(self.db.part_token_offset[wl.P].item())

    def enqueue(self, phase="dedup", i=0):
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


def dedup_report(wl):
    p = DedupPath(wl)
    b = dedup_bytes(wl, p.N, p.M)
    g = p.capture("dedup_step", 50)
    us = float(np.median(p.timed([g], 50, 20)))
    g.destroy()
    g = p.capture("dedup", 50)
    us_sep = float(np.median(p.timed([g], 50, 20)))
    g.destroy()
    ph = {k: float(np.median(p.phase_samples(k, samples=10)))
          for k in ("dedup_layout_dispatch", "layout", "dedup_layout", "dedup_dispatch",
                    "combine_partial", "combine_reduce")}
    out = {"workload": wl.name, "E": wl.E, "P": wl.P, "pairs_N": p.N, "copies_M": p.M,
           "us_per_step_graph": round(us, 3),
           "step": "ep_dedup_layout_dispatch + ep_combine_partial + ep_combine_reduce",
           "launches": {"dedup_layout_dispatch": p.db.plan()},
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
    # the source family each phase's kernels are built from
    family = {"dedup_layout_dispatch": "layout_dispatch", "combine_partial": "combine",
              "combine_reduce": "combine", "dedup_layout": "layout"}.get(phase, phase)
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        f = line.split()
        kv = dict(x.split("=", 1) for x in f[2:])
        if f[0] == phase and f[1] == workload:
            if kv.get("source_digest") != B.source_digest(family):
                return None
            return int(float(kv["traffic_bytes"]))
    return None


def cpu_model():
    """The host CPU's model name with its family / model / stepping numbers
    (a virtualised host may report a bare brand name)."""
    info = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" not in line:
                if info:
                    break                    # the first processor's block is enough
                continue
            k, v = (t.strip() for t in line.split(":", 1))
            info.setdefault(k.lower(), v)
    except OSError:
        pass
    name = info.get("model name") or platform.processor() or "unknown"
    ids = [("family", info.get("cpu family")), ("model", info.get("model")),
           ("stepping", info.get("stepping"))]
    ids = ", ".join("%s %s" % (k, v) for k, v in ids if v)
    return "%s (%s)" % (name, ids) if ids else name


def cpu_baseline(wl, d, N, seconds):
    """The oracle as it stands (single-threaded C): three timed runs of full
    steps of the same workload on one host core, each about seconds / 3
    long; the median run's time per step."""
    import oracle
    bytes_step = algo_bytes(wl, N)["step"]

    def one_step():
        lo = oracle.layout(d["idx"], wl.E, wl.P)
        if wl.payload == "fp8":
            oracle.dispatch_fp8(d["x"], lo["row_of_pair"], wl.K)
        else:
            oracle.dispatch_bf16(d["x"], lo["row_of_pair"], wl.K)
        oracle.combine(d["y"], lo["row_of_pair"], d["w"], wl.T, wl.H, wl.K)

    t0 = time.perf_counter()
    one_step()                                   # untimed: loads the library, sizes a run
    first = time.perf_counter() - t0
    per_run = max(2, int(seconds / 3 / max(first, 1e-6)))
    runs = []
    for _ in range(3):
        t0 = time.perf_counter()
        for _ in range(per_run):
            one_step()
        runs.append((time.perf_counter() - t0) / per_run)
    med = float(np.median(runs))
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return {"value": round(bytes_step / med / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "3 runs of %d full steps (layout+dispatch+combine) of %s on one core; median "
                      "run %.2f ms/step" % (per_run, wl.name, med * 1e3),
            "ms_per_step_runs": [round(r * 1e3, 3) for r in runs],
            "nproc": os.cpu_count(), "affinity_cpus": affinity, "cpu_model": cpu_model()}


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
        p.spin()
        e0.record(p.stream)
        bs.step()
        e1.record(p.stream)
        torch.cuda.synchronize()
        if i >= 2:
            times.append(e0.elapsed_time(e1) * 1e3)
    del flush
    return float(np.median(times))


def native_loop(wl, steps=5000):
    """ep_layout_dispatch + ep_combine from C++ (the package's ep_loop program,
    a child process started before this process touches the GPU): enqueued
    directly, and as a one-step graph replayed per step; host and wall
    microseconds per step.  Uses the library's default launch geometry."""
    exe = os.path.join(ROOT, "combine_ep_layout_05_amd", "ep_loop")
    if not os.path.exists(exe):
        return None
    r = subprocess.run([exe, str(wl.T), str(wl.H), str(wl.K), str(wl.E), str(wl.P), wl.payload,
                        str(steps)], capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        return {"error": (r.stderr or r.stdout)[-300:]}
    return json.loads(r.stdout.strip().splitlines()[-1])


def roofline(bytes_per_launch, us_per_launch, kernel, plan, traffic, cache_state, timing):
    achieved = bytes_per_launch / (us_per_launch * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kernel,
            "launches": plan, "bytes_per_launch": bytes_per_launch,
            "us_per_launch": round(us_per_launch, 3), "cache_state": cache_state,
            "timing": timing}


def large_leg(name, graph_steps, min_steps=100, min_ms=50.0):
    """A bandwidth-bound workload: graphs of `graph_steps` steps, enough samples
    for >= min_steps steps and >= min_ms of timed work."""
    from workloads import WORKLOADS
    wl = WORKLOADS[name]
    p = Path(wl)
    b = algo_bytes(wl, p.N)
    g = p.capture("step", graph_steps)
    est = float(np.median(p.timed([g], graph_steps, 2)))
    samples = max(math.ceil(min_steps / graph_steps),
                  math.ceil(min_ms * 1e3 / (est * graph_steps)))
    v = p.timed([g], graph_steps, samples)
    g.destroy()
    ph = {k: round(float(np.median(p.phase_samples(k, reps=graph_steps, samples=5))), 2)
          for k in ("layout_dispatch", "combine")}
    st = stats(v)
    out = {"us_per_step": st, "timed_steps": graph_steps * samples,
           "timed_ms": round(sum(v) * graph_steps / 1e3, 1),
           "hbm_frac": round(b["step"] / (st["median"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "GBps": round(b["step"] / (st["median"] * 1e-6) / 1e9, 1),
           "phases_us": ph, "launches": p.buf.plan()}
    del p
    return out


def native_ceilings(mib=1024):
    """The package's ep_ceilings probe (hand-written 16-byte-per-lane read,
    write and copy kernels over buffers far larger than the caches), run as a
    child process before this process touches the GPU."""
    exe = os.path.join(ROOT, "combine_ep_layout_05_amd", "ep_ceilings")
    if not os.path.exists(exe):
        return {"error": "ep_ceilings not built"}
    r = subprocess.run([exe, str(mib)], capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        return {"error": (r.stderr or r.stdout)[-300:]}
    return json.loads(r.stdout.strip().splitlines()[-1])


def ceilings(mib=1024, samples=10):
    """HBM read, write and copy rates of this GPU: the native probe's kernels
    (the ceilings), then torch's copy, fill and sum kernels over the same
    sizes for comparison."""
    native = native_ceilings(mib)
    import torch
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    f = a.view(torch.float32)
    s = torch.cuda.Stream()
    res = {}
    for name, fn, nbytes in (("copy", lambda: b.copy_(a), 2 * n), ("write", lambda: b.fill_(3), n),
                             ("read", lambda: f.sum(), n)):
        with torch.cuda.stream(s):
            fn()
        torch.cuda.synchronize()
        v = []
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(samples):
            with torch.cuda.stream(s):
                torch.cuda._sleep(SPIN_CYCLES)
                e0.record(s)
                fn()
                e1.record(s)
            torch.cuda.synchronize()
            v.append(nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        res[name] = {"GBps_median": round(float(np.median(v)), 1), "GBps_max": round(max(v), 1),
                     "bytes": nbytes}
    return {"ceilings": native.get("ceilings_native", native), "torch_kernels": res,
            "buffer_MiB": mib}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="ll_128x7168")
    ap.add_argument("--unfused", action="store_true",
                    help="step = ep_layout + ep_dispatch + ep_combine (default: ep_layout_dispatch + ep_combine)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--default-geometry", action="store_true",
                    help="launch with the library's default geometry, not the tuned rules")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-targets", action="store_true")
    ap.add_argument("--no-dedup", action="store_true")
    ap.add_argument("--no-streamed", action="store_true")
    ap.add_argument("--roofline-only", action="store_true",
                    help="profiling mode: only the per-launch timing the roofline uses (the step's "
                         "two kernels, warm, graphs of 50 launches); prints their roofline")
    ap.add_argument("--ceilings", action="store_true",
                    help="print the plain copy / write / read rates of this GPU and exit")
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
    if args.steps < 1:
        print("--steps must be >= 1", file=sys.stderr)
        sys.exit(2)

    global GEOMETRY
    if args.default_geometry:
        GEOMETRY = None

    if args.ceilings:
        print(json.dumps(ceilings()), flush=True)
        return

    import torch
    from workloads import WORKLOADS
    wl = WORKLOADS[args.workload]

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

    step = "step3" if args.unfused else "step"
    cand = ("dispatch", "combine") if args.unfused else ("layout_dispatch", "combine")
    phase_timing = ("graph of 50 back-to-back launches of the kernel's call, replayed 20 times "
                    "behind a GPU spin; median per launch")

    if args.roofline_only:
        p = Path(wl)
        b = algo_bytes(wl, p.N)
        ph = {k: float(np.median(p.phase_samples(k))) for k in cand}
        plan = p.buf.plan()
        out = {k: roofline(b[k], ph[k], k, plan.get(k), recorded_traffic(k, wl.name), "warm",
                           phase_timing) for k in cand}
        print(json.dumps({"workload": wl.name, "roofline_only": out}), flush=True)
        return

    native = None
    if not args.no_targets:      # before this process initialises the GPU
        native = {w: native_loop(WORKLOADS[w]) for w in (wl.name, "sweep_4x6144", "sweep_8x6144",
                                                         "sweep_16x6144")}

    p = Path(wl)
    b = algo_bytes(wl, p.N)
    v, timing, vk, timing_k = headline(p, args.steps, args.warmup, step)
    st = stats(v)
    us = st["median"]
    phases = {ph: float(np.median(p.phase_samples(ph)))
              for ph in ("layout_dispatch", "layout", "dispatch", "combine")}
    dom = max(cand, key=lambda ph: phases[ph])
    plan = p.buf.plan()
    roof = roofline(b[dom], phases[dom], dom, plan.get(dom), recorded_traffic(dom, wl.name),
                    "warm", phase_timing)
    value = b["step"] / (us * 1e-6) / 1e9

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "value_kind": "cache-warm GB/s: algorithmic bytes per step / device time per step, the "
                      "step's working set resident in L2 and the memory-side cache (see "
                      "hbm_streamed for the same step with nothing cached)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6),
        "us_per_step": us,
        "us_per_step_stats": st,
        "us_per_step_samples_of_steps": dict(stats(vk), timing=timing_k),
        "peak_frac": round(value / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "payload": "fp8_e4m3fn+fp32 per-128 scales dispatch, bf16 combine" if wl.payload == "fp8"
        else "bf16 dispatch, bf16 combine",
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens": wl.T, "hidden": wl.H, "experts": wl.E,
                   "partitions": wl.P, "topk": wl.K, "valid_pairs": p.N,
                   "cache_state": "warm (working set %.1f MB, reused every step)" % (b["step"] / 1e6),
                   "timing": timing,
                   "step": "ep_layout + ep_dispatch + ep_combine" if args.unfused
                   else "ep_layout_dispatch + ep_combine",
                   "parallelism": "single GPU (partitions stand in for EP ranks)",
                   "geometry": {"source": "tuned rules" if GEOMETRY else "library default",
                                **plan}},
        "bytes_per_step": b["step"],
        "phases_us": {k: round(v_, 3) for k, v_ in phases.items()},
        "eager_us_per_step": round(p.eager(500, 20, step), 3),
        "eager_bound_us_per_step": round(p.eager(500, 20, bound=True), 3) if step == "step" else None,
        "graph1_us_per_step": round(p.graph1(1000, step), 3),
        "single_step_us": {"warm": round(single_step_us(p, 50, 0), 3),
                           "cold_after_512MB_write": round(single_step_us(p, 50, 512 << 20), 3)},
        "roofline": roof,
    }
    del p

    if not args.no_streamed:
        vs, phs, set_bytes = streamed(wl)
        sst = stats(vs)
        res["hbm_streamed"] = {
            "us_per_step": sst, "GBps": round(b["step"] / (sst["median"] * 1e-6) / 1e9, 1),
            "frac": round(b["step"] / (sst["median"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "sets": STREAM_SETS, "bytes_rotated": set_bytes,
            "timing": "graphs of 48 steps rotating over %d input/output sets (%.0f MB, above the "
                      "256 MB memory-side cache), %d samples behind a GPU spin; median" % (
                          STREAM_SETS, set_bytes / 1e6, sst["samples"]),
            "phases_us": {k: round(v_, 3) for k, v_ in phs.items()}}
        domh = max(cand, key=lambda ph: phs.get(ph, 0.0))
        res["roofline_hbm_streamed"] = roofline(
            b[domh], phs[domh], domh, plan.get(domh), None, "streamed",
            "graph of 48 launches rotating over %d sets, replayed 10 times behind a GPU spin; "
            "median per launch" % STREAM_SETS)

    if not args.no_targets:
        tg = {"native_loop": native}
        for tt in (4, 8, 16):
            name = "sweep_%dx6144" % tt
            pw = Path(WORKLOADS[name])
            g = pw.capture("step", 100)
            dev = stats(pw.timed([g], 100, 10))
            g.destroy()
            tg[name] = {"device_us_per_step": dev, "graph1_us_per_step": round(pw.graph1(1000), 3),
                        "eager_bound_us_per_step": round(pw.eager(500, 20, bound=True), 3),
                        "launches": pw.buf.plan()}
            if tt == 4:
                tg[name]["eager_us_per_step"] = round(pw.eager(500, 20), 3)
                g = pw.capture("step3", 100)
                tg[name]["unfused_device_us_per_step"] = stats(pw.timed([g], 100, 10))
                g.destroy()
            del pw
        n4 = (native or {}).get("sweep_4x6144") or {}
        tg["sweep_4x6144_target_us"] = 15.0
        tg["sweep_4x6144_end_to_end"] = {
            "graph1_python_us": tg["sweep_4x6144"]["graph1_us_per_step"],
            "graph1_native_us": n4.get("graph1_events_us_per_step"),
            "direct_native_us": n4.get("wall_us_per_step"),
            "device_only_us": tg["sweep_4x6144"]["device_us_per_step"]["median"]}
        tg["bw_4096x7168_zipf"] = large_leg("bw_4096x7168_zipf", 10)
        tg["bw_4096x7168_zipf"]["target_frac"] = 0.60
        tg["masked_16384x4096_bf16"] = large_leg("masked_16384x4096_bf16", 5)
        res["targets"] = tg

    if not args.no_dedup:
        res["dedup"] = [dedup_report(wl),
                        dedup_report(wl.with_(name=wl.name + "_e32p8", E=32, P=8))]

    if not args.no_cpu_baseline:
        from workloads import generate
        d = generate(wl)
        res["cpu_baseline"] = cpu_baseline(wl, d, d["N"], args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
