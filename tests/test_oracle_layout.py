"""Pins of the oracle's layout (counts, scans, deterministic slots).

Pinned by a hand-worked example, by a stable-sort brute force on thousands of
small random cases (masks, duplicate ids, ids >= E), and by invariants on the
full-size workloads.
"""
import json
import os

import numpy as np
import pytest

import oracle
from tests.helpers import brute_layout
from workloads import WORKLOADS, generate

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
KEYS = ("expert_count", "expert_offset", "part_count", "part_offset", "row_of_pair", "src_pair")


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "layout_small.json")))
    out = oracle.layout(np.array(g["topk_idx"], np.int32), g["E"], g["P"])
    for k in KEYS:
        np.testing.assert_array_equal(out[k], g[k], err_msg=k)
    assert int(out["status"][0]) == g["status"]


def _random_case(rng):
    T = int(rng.integers(0, 9))
    K = int(rng.integers(1, 5))
    P = int(rng.integers(1, 5))
    L = int(rng.integers(1, 5))
    E = P * L
    idx = rng.integers(-2, E + 2, size=(T, K)).astype(np.int32)   # masks, bad ids, duplicates
    return idx, E, P


def test_brute_force_random_small_cases():
    rng = np.random.default_rng(1234)
    for _ in range(3000):
        idx, E, P = _random_case(rng)
        got = oracle.layout(idx, E, P)
        ref = brute_layout(idx, E, P)
        for k in KEYS:
            np.testing.assert_array_equal(got[k], ref[k], err_msg="%s idx=%s E=%d P=%d" % (k, idx.tolist(), E, P))
        assert int(got["status"][0]) == int(ref["status"][0])


def check_invariants(idx, E, P, out):
    """I1-I4, I11 of the layout."""
    flat = idx.reshape(-1).astype(np.int64)
    n = flat.size
    valid = (flat >= 0) & (flat < E)
    N = int(out["expert_offset"][E])
    cnt, off = out["expert_count"], out["expert_offset"]
    # I1: counts sum to the number of valid entries (T*K minus masked and bad)
    assert cnt.sum() == N == np.count_nonzero(valid)
    assert np.all(off[1:] - off[:-1] == cnt) and off[0] == 0
    # I2: src_pair is a bijection from [0, N) onto the valid entries, inverse of row_of_pair
    rop, src = out["row_of_pair"], out["src_pair"]
    assert np.all(rop[~valid] == -1)
    assert np.all(src[N:] == -1)
    assert np.array_equal(np.sort(src[:N]), np.nonzero(valid)[0])
    assert np.all(rop[src[:N]] == np.arange(N))
    # I3: within an expert, rows are in increasing (t,k) order and lie in the expert's range
    e_of_row = flat[src[:N]]
    assert np.all(np.diff(e_of_row) >= 0)
    same = e_of_row[1:] == e_of_row[:-1]
    assert np.all(np.diff(src[:N])[same] > 0)
    # I4: partitions are contiguous blocks of experts
    L = E // P
    assert np.array_equal(out["part_offset"][:P], off[0:E:L])
    assert out["part_offset"][P] == N
    assert np.array_equal(out["part_count"], cnt.reshape(P, L).sum(axis=1))
    assert int(out["status"][0]) == int(np.any(flat >= E))


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_invariants_on_workloads(name):
    wl = WORKLOADS[name]
    d = generate(wl, with_x=False, with_y=False)
    out = oracle.layout(d["idx"], wl.E, wl.P)
    check_invariants(d["idx"], wl.E, wl.P, out)
    assert int(out["expert_offset"][wl.E]) == d["N"]


def test_e_equals_p_gives_part_counts_equal_expert_counts():
    # I11
    rng = np.random.default_rng(5)
    idx = rng.integers(-1, 16, size=(200, 4)).astype(np.int32)
    out = oracle.layout(idx, 16, 16)
    np.testing.assert_array_equal(out["part_count"], out["expert_count"])


def test_all_masked_and_empty():
    out = oracle.layout(np.full((5, 3), -1, np.int32), 8, 2)
    assert out["expert_offset"][-1] == 0 and np.all(out["row_of_pair"] == -1)
    assert np.all(out["src_pair"] == -1) and out["status"][0] == 0
    out = oracle.layout(np.zeros((0, 8), np.int32), 8, 2)
    assert out["expert_offset"][-1] == 0 and out["row_of_pair"].size == 0


def test_rejects_bad_arguments():
    idx = np.zeros((2, 2), np.int32)
    for E, P in [(6, 4), (0, 1), (2048, 2)]:
        with pytest.raises(oracle.OracleError):
            oracle.layout(idx, E, P)
    with pytest.raises(oracle.OracleError):
        oracle.layout(np.zeros((2, 17), np.int32), 16, 1)
