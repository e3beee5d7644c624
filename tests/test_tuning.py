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
    assert tu.pick({(1, 0): tail, (2, 0): steady}, incumbent=(4, 0), margin=0.0) == (2, 0)


def test_tie_breaks_on_the_full_tuple_in_any_visiting_order():
    tu = _tuning()
    res = {(8, 0): [1, 5.0, 5.0], (2, 512): [1, 5.0, 5.0], (2, 256): [1, 5.0, 5.0],
           (4, 0): [1, 6.0, 6.0]}
    picks = set()
    for perm in itertools.permutations(res.items()):
        picks.add(tu.pick(dict(perm), incumbent=(4, 0), margin=0.0))
    assert picks == {(2, 256)}


def test_margin_keeps_the_incumbent_unless_beaten_by_it():
    tu = _tuning()
    res = {(4, 0): [1, 10.0, 10.0], (2, 0): [1, 9.9, 9.9]}
    assert tu.pick(res, incumbent=(4, 0), margin=0.0) == (2, 0)
    assert tu.pick(res, incumbent=(4, 0), margin=0.02) == (4, 0)
    res[(2, 0)] = [1, 9.7, 9.7]
    assert tu.pick(res, incumbent=(4, 0), margin=0.02) == (2, 0)


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
    tu.save_rules({key: {"waves": 2, "max_blocks": 512, "avg_latency_us": 3.0}}, path)
    assert tu.lookup("combine", 128, 7168, 8, "fp8", path) == (2, 512)
    assert tu.lookup("dispatch", 128, 7168, 8, "fp8", path) is None
    assert tu.lookup("combine", 129, 7168, 8, "fp8", path) is None
    assert json.load(open(path))["arch"] == "gfx950"
    with pytest.raises(ValueError):
        tu.rule_key("layout", 1, 1, 1, "fp8")


def test_shipped_rules_are_valid_geometries():
    tu = _tuning()
    for key, r in tu.load_rules().items():
        assert key.split(":")[0] in tu.PHASES
        assert (int(r["waves"]), int(r["max_blocks"])) in tu.candidates() + [tu.DEFAULT]
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
