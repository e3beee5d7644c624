"""CPU checks of the launch-geometry tuner's selection rules (no GPU).

The rules restate the lessons recorded for the MoRI EP tuner (MoRI PR #614,
tuner paragraphs): mean over the kept rounds with round 0 dropped, at least 2
rounds, a relative margin with empty = unset, a full-tuple tie-break that does
not depend on visiting order, and adoption only after an A/B against the
incumbent.
"""
import itertools
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _tuning():
    import combine_ep_layout_05_amd.tuning as tu
    return tu


def test_score_drops_round_zero_and_takes_the_mean():
    tu = _tuning()
    assert tu.score([100.0, 2.0, 4.0]) == 3.0
    with pytest.raises(ValueError):
        tu.score([1.0])


def test_mean_penalises_a_heavy_tail_the_median_would_hide():
    tu = _tuning()
    steady = [9.0] + [5.0] * 9
    tail = [9.0] + [4.8] * 8 + [9.0]          # better median, one bad round
    assert tu.pick({(1, 0, 512): tail, (2, 0, 512): steady}, incumbent=(4, 0, 512),
                   margin=0.0) == (2, 0, 512)


def test_tie_breaks_on_the_full_tuple_in_any_visiting_order():
    tu = _tuning()
    res = {(8, 0, 512): [1, 5.0, 5.0], (2, 512, 512): [1, 5.0, 5.0],
           (2, 256, 1024): [1, 5.0, 5.0], (2, 256, 512): [1, 5.0, 5.0],
           (4, 0, 512): [1, 6.0, 6.0]}
    picks = set()
    for perm in itertools.permutations(res.items()):
        picks.add(tu.pick(dict(perm), incumbent=(4, 0, 512), margin=0.0))
    assert picks == {(2, 256, 512)}


def test_margin_keeps_the_incumbent_unless_beaten_by_it():
    tu = _tuning()
    inc = (4, 0, 512)
    res = {inc: [1, 10.0, 10.0], (2, 0, 512): [1, 9.9, 9.9]}
    assert tu.pick(res, incumbent=inc, margin=0.0) == (2, 0, 512)
    assert tu.pick(res, incumbent=inc, margin=0.02) == inc
    res[(2, 0, 512)] = [1, 9.7, 9.7]
    assert tu.pick(res, incumbent=inc, margin=0.02) == (2, 0, 512)


def test_ab_confirmation():
    tu = _tuning()
    assert tu.confirm([50, 4.0, 4.0], [1, 5.0, 5.0], margin=0.0)
    assert not tu.confirm([1, 5.0, 5.0], [1, 5.0, 5.0], margin=0.0)      # a tie is not a win
    assert not tu.confirm([1, 4.95, 4.95], [1, 5.0, 5.0], margin=0.02)


def test_rules_round_trip_and_lookup(tmp_path):
    tu = _tuning()
    path = str(tmp_path / "rules.json")
    assert tu.lookup("combine", 128, 7168, 8, "fp8", path) is None
    key = tu.rule_key("combine", 128, 7168, 8, "fp8")
    key2 = tu.rule_key("layout_dispatch", 128, 7168, 8, "fp8")
    tu.save_rules({key: {"waves": 2, "max_blocks": 512, "slice_cols": 1024, "avg_latency_us": 3.0},
                   key2: {"waves": 6, "max_blocks": 0, "slice_cols": 0, "avg_latency_us": 4.0}},
                  path)
    assert tu.lookup("combine", 128, 7168, 8, "fp8", path) == (2, 512, 1024)
    assert tu.lookup("layout_dispatch", 128, 7168, 8, "fp8", path) == (6, 0, 0)
    assert tu.lookup("dispatch", 128, 7168, 8, "fp8", path) is None
    assert tu.lookup("combine", 129, 7168, 8, "fp8", path) is None
    assert json.load(open(path))["arch"] == "gfx950"
    with pytest.raises(ValueError):
        tu.rule_key("layout", 1, 1, 1, "fp8")
    # a rule written before the slice knob existed reads as 512 columns
    tu.save_rules({key: {"waves": 8, "max_blocks": 256, "avg_latency_us": 3.0}}, path)
    assert tu.lookup("combine", 128, 7168, 8, "fp8", path) == (8, 256, 512)


@pytest.mark.parametrize("phase", ["layout_dispatch", "dedup_layout_dispatch"])
def test_candidates_cover_every_knob_and_only_accepted_fused_sizes(phase):
    """dispatch / combine: every waves x cap x slice combination; the fused
    phases on a fused batch: exactly the workgroup sizes the library's plan
    accepts for that batch (checked through the host-only plan queries)."""
    tu = _tuning()
    import combine_ep_layout_05_amd as ep
    mc = tu.candidates("combine")
    assert len(mc) == len(set(mc)) == 4 * 5 * 2 and (4, 0, 512) in mc and (8, 2048, 1024) in mc
    plan_of = ep.ep_layout_dispatch_plan if phase == "layout_dispatch" else \
        ep.ep_dedup_layout_dispatch_plan
    for sh in tu.PRESETS["bench"]:
        c = tu.candidates(phase, sh)
        plan = plan_of(sh["T"], sh["H"], sh["K"], sh["E"], sh["P"], sh["payload"])
        if plan["kernel"] == "layout_then_dispatch":
            assert c == tu.move_candidates()
            continue
        assert c and all(g[1:] == (0, 0) for g in c)
        for w in (1, 2, 3, 4, 5, 6, 7, 8, 16):
            try:
                plan_of(sh["T"], sh["H"], sh["K"], sh["E"], sh["P"], sh["payload"], (w, 0, 0))
                ok = True
            except ep.EpError:
                ok = False
            assert ok == ((w, 0, 0) in c), (sh["name"], w)
        assert (plan["waves"], 0, 0) in c       # the library's own choice is among them


def test_dedup_candidates_at_the_bench_shapes():
    """The dedup phase's fused sizes: at hidden 7168 (14 steps per token) the
    counting kernel only takes 7 waves, the general kernel 4 or 8; at 4 tokens
    x 6144 (12 steps, 32 entries) the counting kernel takes 6, the general
    kernel 4 or 8."""
    tu = _tuning()
    ll = next(sh for sh in tu.PRESETS["bench"] if sh["name"] == "ll_128x7168")
    assert tu.candidates("dedup_layout_dispatch", ll) == [(4, 0, 0), (7, 0, 0), (8, 0, 0)]
    s4 = next(sh for sh in tu.PRESETS["bench"] if sh["name"] == "sweep_4x6144")
    assert tu.candidates("dedup_layout_dispatch", s4) == [(4, 0, 0), (6, 0, 0), (8, 0, 0)]


def test_plan_reports_the_kernel_each_batch_runs():
    import combine_ep_layout_05_amd as ep
    assert ep.ep_layout_dispatch_plan(4, 6144, 8, 256, 16, "fp8")["kernel"] == "fused_tiny"
    p = ep.ep_layout_dispatch_plan(128, 7168, 8, 288, 16, "fp8")
    assert p == {"kernel": "fused_count", "waves": 7, "blocks": 257, "slice_cols": 512}
    assert ep.ep_layout_dispatch_plan(200, 7168, 8, 288, 16, "fp8")["kernel"] == "fused_general"
    p = ep.ep_layout_dispatch_plan(4096, 7168, 8, 256, 8, "fp8", (2, 0, 1024))
    assert p == {"kernel": "layout_then_dispatch", "waves": 2, "max_blocks": 0, "slice_cols": 1024}
    # the fused kernels take no cap and no 1024-column slice; 3 waves is no kernel's size
    for g in ((4, 256, 0), (4, 0, 1024), (3, 0, 0)):
        with pytest.raises(ep.EpError):
            ep.ep_layout_dispatch_plan(128, 7168, 8, 288, 16, "fp8", g)


def test_shipped_rules_are_valid_geometries():
    tu = _tuning()
    import combine_ep_layout_05_amd as ep
    for key, r in tu.load_rules().items():
        phase = key.split(":")[0]
        assert phase in tu.PHASES
        g = tu.rule_geometry(r)
        if phase in tu.FUSED_PHASES:
            f = dict(kv.split("=") for kv in key.split(":")[1:4])
            shape = next(sh for sh in tu.PRESETS["bench"]
                         if (sh["T"], sh["H"], sh["K"]) == (int(f["T"]), int(f["H"]), int(f["K"])))
            cands = tu.candidates(phase, shape)
            assert g in cands or (g[0], g[1], 0) in cands, key
        else:
            assert g in tu.candidates(phase) + [tu.DEFAULT[phase]], key
        assert r["avg_latency_us"] <= r["incumbent_latency_us"]


def _import_with(env):
    e = dict(os.environ, **env)
    return subprocess.run([sys.executable, "-c", "import combine_ep_layout_05_amd.tuning as t; "
                           "print(t.ROUNDS, t.MARGIN)"], cwd=ROOT, env=e, capture_output=True,
                          text=True)


def test_env_knobs_validated_at_import():
    r = _import_with({"EP_TUNING_ROUNDS": "1"})
    assert r.returncode != 0 and "must be >= 2" in r.stderr
    r = _import_with({"EP_TUNING_ROUNDS": "", "EP_TUNING_MARGIN": ""})      # empty = unset
    assert r.returncode == 0 and r.stdout.split() == ["10", "0.0"]
    r = _import_with({"EP_TUNING_MARGIN": "1.5"})
    assert r.returncode != 0 and "[0, 1)" in r.stderr


def test_presets_time_the_bench_workloads():
    """Every preset shape names the bench workload whose inputs it is timed
    on, with that workload's exact shape."""
    from workloads import WORKLOADS
    tu = _tuning()
    for sh in tu.PRESETS["bench"]:
        wl = WORKLOADS[sh["workload"]]
        assert (wl.T, wl.H, wl.K, wl.E, wl.P, wl.payload) == \
            (sh["T"], sh["H"], sh["K"], sh["E"], sh["P"], sh["payload"]), sh["name"]


def test_workload_inputs():
    import numpy as np
    tu = _tuning()
    assert tu.workload_inputs(None, 4, 1024, 8, 32, 8, "fp8") is None
    d = tu.workload_inputs("tiny_4x1024", 4, 1024, 8, 32, 8, "fp8")
    assert d["idx"].shape == (4, 8) and d["x"].shape == (4, 1024) and d["y"].shape == (32, 1024)
    assert d["idx"].dtype == np.int32 and d["x"].dtype == np.uint16
    with pytest.raises(ValueError):
        tu.workload_inputs("tiny_4x1024", 4, 1024, 8, 64, 8, "fp8")
