"""CPU checks of the benchmark's host logic: the algorithmic byte counts, the
gate that keeps counter readings to the sources they were taken from, the
one-GPU refusal and the CPU description beside the oracle baseline."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import WORKLOADS  # noqa: E402


def test_algorithmic_bytes_of_the_five_configurations():
    """fp8 dispatch T*2H + N*(H + H/32), bf16 dispatch T*2H + N*2H, combine
    N*2H + T*2H, worked out by hand for each configuration (N = valid pairs:
    every entry, except the 13107 masked ones of the 16384-token batch)."""
    cases = {  # workload: (N, dispatch bytes, combine bytes)
        "tiny_4x1024": (32, 41984, 73728),
        "ll_128x7168": (1024, 9404416, 16515072),
        "sweep_4x6144": (32, 251904, 442368),
        "sweep_16x6144": (128, 1007616, 1769472),
        "bw_4096x7168_zipf": (32768, 300941312, 528482304),
        "masked_16384x4096_bf16": (117965, 1100587008, 1100587008),
    }
    for name, (n, disp, comb) in cases.items():
        a = bench.algo_bytes(WORKLOADS[name], n)
        assert (a["dispatch"], a["layout_dispatch"], a["combine"]) == (disp, disp, comb), name
        assert a["step"] == disp + comb and a["layout"] == 0


def test_recorded_traffic_follows_the_source_digest(tmp_path, monkeypatch):
    """A committed reading is returned exactly when its digest matches the
    current sources of its kernel family (else None, and the bench reports
    no traffic); an unknown pair and a missing file give None."""
    from combine_ep_layout_05_amd import build as B
    family = {"dedup_layout_dispatch": "layout_dispatch", "combine_partial": "combine",
              "combine_reduce": "combine", "dedup_layout": "layout"}
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    lines = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    assert len(lines) >= 13
    for f in lines:
        kv = dict(x.split("=", 1) for x in f[2:])
        current = kv["source_digest"] == B.source_digest(family.get(f[0], f[0]))
        want = int(float(kv["traffic_bytes"])) if current else None
        assert bench.recorded_traffic(f[0], f[1]) == want, f[:2]
    assert bench.recorded_traffic("combine", "no_such_workload") is None
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "traffic.txt").write_text(
        "combine ll_128x7168 traffic_bytes=123 source_digest=00\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_traffic("combine", "ll_128x7168") is None
    monkeypatch.setattr(bench, "ROOT", str(tmp_path / "nowhere"))
    assert bench.recorded_traffic("combine", "ll_128x7168") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "one GPU only" in r.stderr
    assert r.stdout == ""


def test_stats_and_cpu_description():
    st = bench.stats([3.0, 1.0, 2.0])
    assert st == {"mean": 2.0, "median": 2.0, "min": 1.0, "samples": 3}
    m = bench.cpu_model()
    assert isinstance(m, str) and m and m != "unknown"
