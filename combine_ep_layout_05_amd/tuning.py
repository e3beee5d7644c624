"""Launch-geometry tuner for ep_layout_dispatch, ep_dispatch and ep_combine on MI355X.

A geometry is (waves_per_block, max_blocks, slice_cols):
  - dispatch / combine: 1, 2, 4 or 8 waves per workgroup; one wave per work
    item (max_blocks = 0) or a cap on the number of workgroups, whose waves
    then stride over the items; 512 or 1024 columns of one token per item;
  - layout_dispatch: for batches that run fused (one launch, T*K <= 4096)
    the fused kernel's waves per workgroup, the sizes that kernel takes
    (found with ep_layout_dispatch_plan), max_blocks 0 and slice 0; for
    larger batches the dispatch kernel's geometry as above.  (0, 0, 0) is
    the library's own choice;
  - dedup_layout_dispatch: the same for ep_dedup_layout_dispatch (sizes from
    ep_dedup_layout_dispatch_plan).
The inputs are those of the bench's synthetic workload of each shape (its
routing, masked entries and outlier rows; a preset entry names it), when the
repository's `workloads` package is importable, else uniform routing with
nothing masked: the best geometry moves with the input, e.g. at 16384 x 4096
bf16 one capped-grid dispatch won by 2.8 % on unmasked inputs and lost by 2 %
with the workload's 10 % of entries masked.
Candidates of the calls a step is made of are timed inside that step, in
the context they run in: a layout_dispatch or combine candidate in the plain
step (ep_layout_dispatch, then ep_combine reading the row map it has just
written; the other call with its saved rule, else the library's choice), a
dedup_layout_dispatch candidate in the per-destination step (then
ep_combine_partial and ep_combine_reduce).  Their scores are step times.
(Timed alone, on a row map written long before, the best combine geometry at
128 x 7168 was slower in the step than the library default.)  A dispatch
candidate, for bare ep_dispatch calls, is timed alone.
Outputs do not depend on it; time does, and the best choice moves with token
count and phase.  The selection rules follow what the MoRI EP tuner learned
(MoRI PR #614 "perf(ep): InterNodeV1LL low-token latency on MI300X + CX7",
tuner paragraphs):

  - score a candidate by its MEAN latency over the kept rounds; round 0 is
    dropped as warm-up.  The mean, unlike the median, is pulled up by a
    heavy tail, which is what a geometry that contends for the CUs shows;
  - at least 2 rounds (one is dropped): EP_TUNING_ROUNDS below 2 is rejected
    when this module is imported, with a message that says why;
  - one relative margin (EP_TUNING_MARGIN, default 0: any improvement wins)
    decides both whether a candidate displaces the incumbent and whether a
    saved rule may be replaced; an empty variable counts as unset;
  - ties break on the full geometry tuple, so the pick does not depend on the
    order in which the sweep visits candidates;
  - a pick is adopted only after an interleaved A/B re-measurement against
    the incumbent (the saved rule for the shape, else the library default;
    with --fresh always the library default) confirms it, so a single noisy
    sample cannot win.

Rules are kept in a JSON file (tuned_geometry.json beside this module by
default), keyed by phase and exact shape; EpBuffers(..., geometry="tuned")
and EpDedupBuffers(..., geometry="tuned") use them.  Run the sweep on the GPU with
    python -m combine_ep_layout_05_amd.tuning --preset bench --write
(`--fresh` re-tunes every shape of the given phases against the library
default and replaces those phases' rules by the ones adopted in that run, so
rules that no longer win by the margin are dropped).
"""
from __future__ import annotations

import argparse
import json
import os
import sys


def _env_rounds():
    raw = os.environ.get("EP_TUNING_ROUNDS") or "10"
    try:
        n = int(raw)
    except ValueError:
        raise ValueError("EP_TUNING_ROUNDS=%r is not an integer" % raw) from None
    if n < 2:
        raise ValueError("EP_TUNING_ROUNDS=%d: must be >= 2, because round 0 is dropped as "
                         "warm-up and the score needs at least one kept round" % n)
    return n


def _env_margin():
    raw = os.environ.get("EP_TUNING_MARGIN") or "0.0"
    try:
        m = float(raw)
    except ValueError:
        raise ValueError("EP_TUNING_MARGIN=%r is not a number" % raw) from None
    if not 0.0 <= m < 1.0:
        raise ValueError("EP_TUNING_MARGIN=%g: must be in [0, 1)" % m)
    return m


ROUNDS = _env_rounds()
MARGIN = _env_margin()
VERBOSE = (os.environ.get("EP_TUNING_VERBOSE") or "0") not in ("0", "")

PHASES = ("layout_dispatch", "dispatch", "combine", "dedup_layout_dispatch")
FUSED_PHASES = ("layout_dispatch", "dedup_layout_dispatch")   # fused for small batches
LIBRARY = (0, 0, 0)                   # the library's own choice
# the incumbent of a fresh sweep: the library's own choice (the combine's
# depends on the batch: 2 waves per workgroup when it streams, else 4)
DEFAULT = {"layout_dispatch": LIBRARY, "dispatch": (4, 0, 512), "combine": LIBRARY,
           "dedup_layout_dispatch": LIBRARY}
WAVES = (1, 2, 4, 8)
MAX_BLOCKS = (0, 256, 512, 1024, 2048)
SLICES = (512, 1024)
FUSED_WAVES = (1, 2, 4, 6, 7, 8)       # the workgroup sizes the fused kernels take, all told
RULES_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tuned_geometry.json")


def move_candidates():
    """Geometries of the dispatch and combine kernels."""
    return [(w, b, s) for w in WAVES for b in MAX_BLOCKS for s in SLICES]


def candidates(phase, shape=None):
    """Candidate geometries of a phase; those of the fused phases depend on
    the shape (dict with T, H, K, E, P, payload): the workgroup sizes its
    fused kernel takes, or the dispatch kernel's geometries when the batch is
    not fused."""
    if phase not in PHASES:
        raise ValueError("phase must be one of %s" % (PHASES,))
    if phase not in FUSED_PHASES:
        return move_candidates()
    from . import EpError, ep_dedup_layout_dispatch_plan, ep_layout_dispatch_plan
    plan = ep_layout_dispatch_plan if phase == "layout_dispatch" else ep_dedup_layout_dispatch_plan
    T, H, K, E, P, payload = (shape[k] for k in ("T", "H", "K", "E", "P", "payload"))
    if plan(T, H, K, E, P, payload)["kernel"] == "layout_then_dispatch":
        return move_candidates()
    out = []
    for w in FUSED_WAVES:
        try:
            plan(T, H, K, E, P, payload, (w, 0, 0))
        except EpError:
            continue
        out.append((w, 0, 0))
    return out


# ---- selection (pure functions) ---------------------------------------------

def score(samples):
    """Mean latency of the kept rounds (round 0 dropped)."""
    if len(samples) < 2:
        raise ValueError("need at least 2 rounds, got %d" % len(samples))
    kept = samples[1:]
    return sum(kept) / len(kept)


def beats(new_us, old_us, margin):
    return new_us < old_us * (1.0 - margin)


def pick(results, incumbent, margin=None):
    """results: {geometry tuple: per-round latencies}.  The fastest mean wins,
    ties broken by the smaller geometry tuple; the incumbent (when it was
    measured) is kept unless the winner beats it by the margin."""
    margin = MARGIN if margin is None else margin
    best = min(results, key=lambda g: (score(results[g]), tuple(g)))
    if incumbent in results and best != incumbent and \
            not beats(score(results[best]), score(results[incumbent]), margin):
        return incumbent
    return best


def confirm(new_samples, old_samples, margin=None):
    """A/B decision: adopt the new geometry only if its mean beats the
    incumbent's, measured in the same interleaved rounds, by the margin."""
    margin = MARGIN if margin is None else margin
    return beats(score(new_samples), score(old_samples), margin)


# ---- rules file --------------------------------------------------------------

def rule_key(phase, T, H, K, payload):
    if phase not in PHASES:
        raise ValueError("phase must be one of %s" % (PHASES,))
    return "%s:T=%d:H=%d:K=%d:%s" % (phase, T, H, K, payload)


def load_rules(path=None):
    path = path or RULES_PATH
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        data = json.load(f)
    return data.get("rules", {})


def save_rules(rules, path=None, arch="gfx950"):
    path = path or RULES_PATH
    tmp = path + ".tmp"
    with open(tmp, "w") as f:
        json.dump({"arch": arch, "rules": dict(sorted(rules.items()))}, f, indent=1)
        f.write("\n")
    os.replace(tmp, path)


def rule_geometry(rule):
    """(waves, max_blocks, slice_cols) of a saved rule (slice 512 when absent)."""
    return (int(rule["waves"]), int(rule["max_blocks"]), int(rule.get("slice_cols", 512)))


def lookup(phase, T, H, K, payload, path=None):
    """Saved geometry for this exact shape, or None (library default)."""
    r = load_rules(path).get(rule_key(phase, T, H, K, payload))
    return None if r is None else rule_geometry(r)


# ---- measurement (GPU) ---------------------------------------------------------

SPIN_CYCLES = 200000                  # GPU spin ahead of a timed graph (about 80 us)


def workload_inputs(name, T, H, K, E, P, payload):
    """The seeded inputs of the named synthetic workload (the repository's
    `workloads` package, beside this one), or None when no name is given or
    that package is not importable.  The workload must have this shape."""
    if not name:
        return None
    try:
        from workloads import WORKLOADS, generate
    except ImportError:
        return None
    wl = WORKLOADS[name]
    if (wl.T, wl.H, wl.K, wl.E, wl.P, wl.payload) != (T, H, K, E, P, payload):
        raise ValueError("workload %s is not the shape T=%d H=%d K=%d E=%d P=%d %s"
                         % (name, T, H, K, E, P, payload))
    return generate(wl)


class ShapeBench:
    """Seeded synthetic inputs and persistent buffers for one shape; times
    one phase under a given geometry from HIP graphs of back-to-back
    launches (device time per launch: a GPU spin ahead of the first event
    keeps the host's graph-launch time out of the timed region)."""

    def __init__(self, T, H, K, E, P, payload="fp8", seed=0, launches=20, workload=None):
        import torch
        from . import EpBuffers
        self.torch = torch
        self.T, self.H, self.K, self.E, self.P, self.payload = T, H, K, E, P, payload
        self.dbuf = None                  # per-destination buffers, made on first use
        self.launches = launches
        dev = "cuda"
        d = workload_inputs(workload, T, H, K, E, P, payload)
        if d is not None:
            # the named workload's own inputs: its routing, masked entries and
            # outlier rows, as the bench times them
            import numpy as np

            def up(a, bf16=False):
                t = torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if bf16 else a))
                return (t.view(torch.bfloat16) if bf16 else t).to(dev)
            self.idx, self.w = up(d["idx"]), up(d["w"])
            self.x, self.y = up(d["x"], True), up(d["y"], True)
        else:
            g = torch.Generator().manual_seed(seed)
            idx = torch.rand(T, E, generator=g).argsort(dim=1)[:, :K].to(torch.int32)
            w = torch.softmax(torch.randn(T, K, generator=g), dim=1)
            self.idx = idx.contiguous().to(dev)
            self.w = w.contiguous().to(dev)
            self.x = torch.randn(T, H, generator=g).to(torch.bfloat16).to(dev)
            self.y = torch.randn(T * K, H, generator=g).to(torch.bfloat16).to(dev)
        self.buf = EpBuffers(T, H, K, E, P, payload=payload)
        self.stream = torch.cuda.Stream()
        self.buf.layout(self.idx, self.stream)
        torch.cuda.synchronize()
        self.graphs = {}

    def _enqueue(self, phase, geometry):
        from . import EpDedupBuffers, ep_combine, ep_dispatch, ep_layout_dispatch
        b = self.buf
        saved = lambda ph: lookup(ph, self.T, self.H, self.K, self.payload)
        if phase in ("layout_dispatch", "combine"):
            # the plain step: layout+dispatch writes the row map the combine reads
            ld = geometry if phase == "layout_dispatch" else saved("layout_dispatch")
            ep_layout_dispatch(self.idx, self.x, b.E, b.P, b.payload, b.expert_count,
                               b.expert_offset, b.part_count, b.part_offset, b.row_of_pair,
                               b.src_pair, b.status, b.ws, b.recv_x, b.recv_scales, self.stream,
                               None if ld is None or tuple(ld) == LIBRARY else ld)
            cb = geometry if phase == "combine" else saved("combine")
            ep_combine(self.y, b.row_of_pair, self.w, b.out, self.stream,
                       None if cb is None or tuple(cb) == LIBRARY else cb)
        elif phase == "dedup_layout_dispatch":
            # the per-destination step
            if self.dbuf is None:
                self.dbuf = EpDedupBuffers(self.T, self.H, self.K, self.E, self.P, self.payload)
            db = self.dbuf
            db.layout_dispatch(self.idx, self.x, b, self.stream,
                               None if tuple(geometry) == LIBRARY else geometry)
            db.combine_partial(self.y, b.row_of_pair, self.w, self.stream)
            db.combine_reduce(self.stream)
        else:
            ep_dispatch(self.x, self.K, b.row_of_pair, b.payload, b.recv_x, b.recv_scales,
                        self.stream, geometry)

    def graph(self, phase, geometry):
        from . import ep_graph_begin, ep_graph_end
        key = (phase, geometry)
        if key not in self.graphs:
            with self.torch.cuda.stream(self.stream):
                ep_graph_begin(self.stream)
                for _ in range(self.launches):
                    self._enqueue(phase, geometry)
                self.graphs[key] = ep_graph_end(self.stream)
        return self.graphs[key]

    def round_us(self, phase, geometry):
        torch = self.torch
        g = self.graph(phase, geometry)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(self.stream):
            torch.cuda._sleep(SPIN_CYCLES)
        e0.record(self.stream)
        g.launch(self.stream)
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / self.launches

    def sweep(self, phase, geometries, rounds):
        return {geom: [self.round_us(phase, geom) for _ in range(rounds)] for geom in geometries}

    def ab(self, phase, new, old, rounds):
        """Interleaved rounds new, old, new, old, ..."""
        a, b = [], []
        for _ in range(rounds):
            a.append(self.round_us(phase, new))
            b.append(self.round_us(phase, old))
        return a, b

    def close(self):
        for g in self.graphs.values():
            g.destroy()
        self.graphs.clear()


def tune(phase, shape, rules, rounds=None, margin=None, fresh=False, log=print):
    """Sweep one phase on one shape; returns (rule or None, report dict).
    The incumbent is the saved rule for the shape, else (and always with
    fresh) the library default."""
    rounds = ROUNDS if rounds is None else rounds
    margin = MARGIN if margin is None else margin
    T, H, K, E, P, payload = (shape[k] for k in ("T", "H", "K", "E", "P", "payload"))
    key = rule_key(phase, T, H, K, payload)
    saved = None if fresh else rules.get(key)
    incumbent = DEFAULT[phase] if saved is None else rule_geometry(saved)
    sb = ShapeBench(T, H, K, E, P, payload, seed=shape.get("seed", 0),
                    workload=shape.get("workload"))
    try:
        cands = candidates(phase, shape)
        if incumbent not in cands:
            cands.append(incumbent)
        res = sb.sweep(phase, cands, rounds)
        if VERBOSE:
            for g in sorted(res, key=lambda g: score(res[g])):
                log("  %s %s %s mean %.3f us rounds %s" % (
                    phase, key, g, score(res[g]), ["%.2f" % v for v in res[g]]))
        best = pick(res, incumbent, margin)
        report = {"key": key, "incumbent": list(incumbent), "sweep_pick": list(best),
                  "candidates": len(cands), "sweep_mean_us": round(score(res[best]), 4),
                  "incumbent_sweep_mean_us": round(score(res[incumbent]), 4)}
        if best == incumbent:
            report["adopted"] = False
            return None, report
        new_s, old_s = sb.ab(phase, best, incumbent, rounds)
        ok = confirm(new_s, old_s, margin)
        report.update(ab_new_us=round(score(new_s), 4), ab_old_us=round(score(old_s), 4),
                      adopted=bool(ok))
        if not ok:
            return None, report
        rule = {"waves": best[0], "max_blocks": best[1], "slice_cols": best[2],
                "avg_latency_us": round(score(new_s), 4), "incumbent": list(incumbent),
                "incumbent_latency_us": round(score(old_s), 4), "rounds": rounds,
                "margin": margin}
        return rule, report
    finally:
        sb.close()


PRESETS = {
    "bench": [
        dict(name="ll_128x7168", T=128, H=7168, K=8, E=288, P=16, payload="fp8",
             workload="ll_128x7168"),
        dict(name="sweep_4x6144", T=4, H=6144, K=8, E=256, P=16, payload="fp8",
             workload="sweep_4x6144"),
        dict(name="sweep_8x6144", T=8, H=6144, K=8, E=256, P=16, payload="fp8",
             workload="sweep_8x6144"),
        dict(name="sweep_16x6144", T=16, H=6144, K=8, E=256, P=16, payload="fp8",
             workload="sweep_16x6144"),
        dict(name="bw_4096x7168", T=4096, H=7168, K=8, E=256, P=8, payload="fp8",
             workload="bw_4096x7168_zipf"),
        dict(name="masked_16384x4096_bf16", T=16384, H=4096, K=8, E=128, P=8, payload="bf16",
             workload="masked_16384x4096_bf16"),
    ],
}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--preset", default="bench", choices=sorted(PRESETS))
    ap.add_argument("--phases", default=",".join(PHASES))
    ap.add_argument("--rules", default=None, help="rules file (default: the package's)")
    ap.add_argument("--write", action="store_true", help="save adopted rules")
    ap.add_argument("--fresh", action="store_true",
                    help="tune the given phases against the library default and replace their "
                         "saved rules by this run's adopted ones (rules that no longer win by "
                         "the margin are dropped); other phases' rules are kept")
    args = ap.parse_args(argv)
    rules = load_rules(args.rules)
    phases = [p for p in args.phases.split(",") if p]
    for p in phases:
        if p not in PHASES:
            raise SystemExit("unknown phase %r" % p)
    print("rounds %d (round 0 dropped), margin %g, %s" % (
        ROUNDS, MARGIN, "fresh: incumbent = library default" if args.fresh else
        "incumbent = saved rule, else library default"), flush=True)
    # --fresh: drop the saved rules of the phases being tuned, keep the others
    new_rules = {k: v for k, v in rules.items()
                 if not (args.fresh and k.split(":")[0] in phases)}
    for shape in PRESETS[args.preset]:
        for phase in phases:
            rule, rep = tune(phase, shape, rules, fresh=args.fresh)
            print(json.dumps(rep), flush=True)
            if rule is not None:
                new_rules[rep["key"]] = rule
    if args.write:
        save_rules(new_rules, args.rules)
        print("rules written to %s" % (args.rules or RULES_PATH), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
