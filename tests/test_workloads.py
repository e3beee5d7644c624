"""Generator checks: determinism, routing structure, masks, skew, weights."""
import numpy as np
import pytest

from workloads import WORKLOADS, generate


@pytest.mark.parametrize("name", ["tiny_4x1024", "ll_128x7168", "sweep_4x6144"])
def test_same_seed_same_bytes(name):
    wl = WORKLOADS[name]
    a, b = generate(wl), generate(wl)
    for k in ("idx", "w", "x", "y"):
        assert np.array_equal(a[k], b[k]), k
    c = generate(wl, seed=wl.seed + 100)
    assert not np.array_equal(a["x"], c["x"])


@pytest.mark.parametrize("name", [n for n in WORKLOADS if WORKLOADS[n].routing == "uniform"])
def test_distinct_ids_and_weights(name):
    wl = WORKLOADS[name]
    d = generate(wl, with_x=False, with_y=False)
    idx = d["idx"]
    assert idx.shape == (wl.T, wl.K) and idx.dtype == np.int32
    for row in idx:
        v = row[row >= 0]
        assert len(set(v.tolist())) == v.size and np.all(v < wl.E)
    w = d["w"]
    valid = idx >= 0
    assert np.all(w[~valid] == 0)
    s = w.sum(axis=1)
    assert np.allclose(s[valid.any(axis=1)], 1.0, atol=1e-5)


def test_masked_count_exact():
    wl = WORKLOADS["masked_16384x4096_bf16"]
    d = generate(wl, with_x=False, with_y=False)
    assert np.count_nonzero(d["idx"] == -1) == round(0.1 * wl.T * wl.K) == 13107
    assert d["N"] == wl.T * wl.K - 13107


def test_zipf_partition0_ratio_and_skew():
    wl = WORKLOADS["bw_4096x7168_zipf"]
    d = generate(wl, with_x=False, with_y=False)
    idx = d["idx"]
    for row in idx[:256]:
        assert len(set(row.tolist())) == wl.K
    load0 = np.count_nonzero(idx < wl.L)
    ratio = load0 / (wl.T * wl.K / wl.P)
    assert abs(ratio - 1.5) <= 0.02
    cnt = np.bincount(idx.reshape(-1), minlength=wl.E)
    assert cnt.max() > 0.5 * wl.T          # the hottest expert is in most tokens


def test_outlier_rows():
    wl = WORKLOADS["ll_128x7168"]
    d = generate(wl, with_y=False)
    rows = d["meta"]["outlier_rows"]
    assert len(rows) == 1
    x = (d["x"].astype(np.uint32) << 16).view(np.float32)
    amax = np.abs(x).max(axis=1)
    assert amax[rows[0]] > 10 * np.median(amax)
