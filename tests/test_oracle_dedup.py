"""Pins of the oracle's per-destination dedup layout and two-level combine.

Pinned by a hand-worked example, a brute force of the token-partition layout
on random small cases, invariants on every workload, a vectorised exact-fmaf
re-evaluation of level 1, sequential fp32 adds for level 2, and the reduction
to the plain combine for tokens whose experts all sit in one partition.
"""
import json
import os

import numpy as np
import pytest

import oracle
from tests.helpers import bf16_to_f32, fmaf_exact_np
from workloads import WORKLOADS, generate
from workloads.gen import to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
KEYS = ("tp_row", "part_tokens", "part_token_offset", "tp_src", "kmask")


def brute_dedup(idx, E, P):
    T, K = idx.shape
    L = E // P
    kmask = np.zeros((T, P), np.uint32)
    for t in range(T):
        for k in range(K):
            e = int(idx[t, k])
            if 0 <= e < E:
                kmask[t, e // L] |= np.uint32(1 << k)
    present = kmask != 0
    tp = np.nonzero(present.reshape(-1))[0]
    order = tp[np.lexsort((tp // P, tp % P))]          # partition major, token ascending
    tp_row = np.full(T * P, -1, np.int64)
    tp_row[order] = np.arange(order.size)
    tp_src = np.full(T * P, -1, np.int64)
    tp_src[:order.size] = order
    part_tokens = present.sum(axis=0)
    return dict(tp_row=tp_row, part_tokens=part_tokens,
                part_token_offset=np.concatenate([[0], np.cumsum(part_tokens)]),
                tp_src=tp_src, kmask=kmask.reshape(-1),
                status=np.array([int(np.any(idx >= E))]))


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "layout_small.json")))
    out = oracle.dedup_layout(np.array(g["topk_idx"], np.int32), g["E"], g["P"])
    for k in KEYS:
        np.testing.assert_array_equal(out[k], g["dedup"][k], err_msg=k)
    assert int(out["status"][0]) == g["dedup"]["status"]


def test_brute_force_random_small_cases():
    rng = np.random.default_rng(4321)
    for _ in range(2000):
        T = int(rng.integers(0, 8))
        K = int(rng.integers(1, 5))
        P = int(rng.integers(1, 5))
        E = P * int(rng.integers(1, 4))
        idx = rng.integers(-2, E + 2, size=(T, K)).astype(np.int32)
        got = oracle.dedup_layout(idx, E, P)
        ref = brute_dedup(idx, E, P)
        for k in KEYS:
            np.testing.assert_array_equal(got[k], ref[k], err_msg="%s %s" % (k, idx.tolist()))
        assert int(got["status"][0]) == int(ref["status"][0])


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_invariants_on_workloads(name):
    wl = WORKLOADS[name]
    d = generate(wl, with_x=False, with_y=False)
    out = oracle.dedup_layout(d["idx"], wl.E, wl.P)
    km = out["kmask"]
    M = int(out["part_token_offset"][-1])
    # every valid entry is in exactly one mask bit; a row per present (token, partition)
    assert sum(bin(int(m)).count("1") for m in km) == d["N"]
    assert M == np.count_nonzero(km) <= d["N"]
    assert np.all(out["tp_src"][M:] == -1)
    assert np.array_equal(np.sort(out["tp_src"][:M]), np.nonzero(km)[0])
    assert np.all(out["tp_row"][out["tp_src"][:M]] == np.arange(M))
    # rows of a partition are contiguous and token-ascending
    p_of_row = out["tp_src"][:M] % wl.P
    assert np.all(np.diff(p_of_row) >= 0)
    same = p_of_row[1:] == p_of_row[:-1]
    assert np.all(np.diff(out["tp_src"][:M] // wl.P)[same] > 0)


def _setup(name, seed=None, T=None):
    wl = WORKLOADS[name] if T is None else WORKLOADS[name].with_(T=T)
    d = generate(wl, seed=seed)
    lo = oracle.layout(d["idx"], wl.E, wl.P)
    dd = oracle.dedup_layout(d["idx"], wl.E, wl.P)
    return wl, d, lo, dd


@pytest.mark.parametrize("name", ["tiny_4x1024", "ll_128x7168"])
def test_two_level_combine_exact(name):
    """Level 1 re-evaluated with the vectorised exact fmaf over each partition's
    entries in k order; level 2 with sequential fp32 adds in partition order."""
    wl, d, lo, dd = _setup(name)
    T, H, K, P = wl.T, wl.H, wl.K, wl.P
    part = oracle.combine_partial(d["y"], lo["row_of_pair"], d["w"], dd["tp_row"], dd["kmask"], T, H, K, P)
    out = oracle.combine_reduce(part, dd["tp_row"], T, H, P)
    rop = lo["row_of_pair"].reshape(T, K)
    yf = bf16_to_f32(d["y"])
    km = dd["kmask"].reshape(T, P)
    tpr = dd["tp_row"].reshape(T, P)
    ref_out = np.zeros((T, H), np.float32)
    for p in range(P):
        acc = np.zeros((T, H), np.float32)
        for k in range(K):
            use = ((km[:, p] >> k) & 1).astype(bool)
            upd = fmaf_exact_np(np.broadcast_to(d["w"][:, k:k + 1], acc.shape), yf[np.maximum(rop[:, k], 0)], acc)
            acc = np.where(use[:, None], upd, acc)
        pres = tpr[:, p] >= 0
        pb = to_bf16_bits(acc)
        np.testing.assert_array_equal(part[tpr[pres, p]], pb[pres], err_msg="partition %d" % p)
        ref_out = np.where(pres[:, None], (ref_out + bf16_to_f32(pb)).astype(np.float32), ref_out)
    np.testing.assert_array_equal(out, to_bf16_bits(ref_out))


def test_single_partition_tokens_equal_plain_combine():
    """A token whose experts all sit in one partition: level 2 adds one
    bf16 partial to +0, so the result is the plain combine's."""
    wl, d, lo, dd = _setup("tiny_4x1024", seed=11, T=64)
    L = wl.E // wl.P
    rng = np.random.default_rng(11)
    idx = d["idx"].copy()
    for t in range(0, wl.T, 2):                     # even tokens: K distinct experts in one partition
        p = int(rng.integers(0, wl.P))
        idx[t] = p * L + rng.permutation(L)[:wl.K] if L >= wl.K else p * L + np.arange(wl.K) % L
    d["idx"] = idx
    lo = oracle.layout(idx, wl.E, wl.P)
    dd = oracle.dedup_layout(idx, wl.E, wl.P)
    plain = oracle.combine(d["y"], lo["row_of_pair"], d["w"], wl.T, wl.H, wl.K)
    part = oracle.combine_partial(d["y"], lo["row_of_pair"], d["w"], dd["tp_row"], dd["kmask"],
                                  wl.T, wl.H, wl.K, wl.P)
    out = oracle.combine_reduce(part, dd["tp_row"], wl.T, wl.H, wl.P)
    single = (dd["kmask"].reshape(wl.T, wl.P) != 0).sum(axis=1) == 1
    assert single[::2].all()
    np.testing.assert_array_equal(out[single], plain[single])


def test_partial_with_every_entry_is_the_plain_combine():
    """Level 1 with one copy per token whose mask holds all K entries --
    masked ones (row -1) included -- is the plain combine: the same fmaf
    sequence over the entries that have a receive row, masked entries
    contributing nothing."""
    wl = WORKLOADS["masked_16384x4096_bf16"].with_(name="partial_all", T=96, H=256)
    d = generate(wl, seed=5)
    lo = oracle.layout(d["idx"], wl.E, wl.P)
    assert (lo["row_of_pair"] < 0).any()
    # every weight nonzero, and a row of ones just before y in memory, so an
    # entry with row -1 that were not skipped would change the sums
    w = np.random.default_rng(5).random((wl.T, wl.K)).astype(np.float32) + 0.5
    ybig = np.empty((d["y"].shape[0] + 1, wl.H), np.uint16)
    ybig[0] = 0x3F80
    ybig[1:] = d["y"]
    y = ybig[1:]
    plain = oracle.combine(y, lo["row_of_pair"], w, wl.T, wl.H, wl.K)
    tp_row = np.arange(wl.T, dtype=np.int32)
    kmask = np.full(wl.T, (1 << wl.K) - 1, np.uint32)
    part = oracle.combine_partial(y, lo["row_of_pair"], w, tp_row, kmask, wl.T, wl.H, wl.K, 1)
    np.testing.assert_array_equal(part, plain)


def test_dedup_dispatch_rows_hold_the_token():
    """Dedup dispatch is the plain fp8 dispatch with one row per (token,
    partition): every row carries its token's quantised bytes and scales."""
    wl, d, lo, dd = _setup("tiny_4x1024")
    rx, rs = oracle.dispatch_fp8(d["x"], lo["row_of_pair"], wl.K)
    drx, drs = oracle.dispatch_fp8(d["x"], dd["tp_row"], wl.P)
    M = int(dd["part_token_offset"][-1])
    t_of_row = dd["tp_src"][:M] // wl.P
    first_row = lo["row_of_pair"].reshape(wl.T, wl.K).max(axis=1)
    np.testing.assert_array_equal(drx[:M], rx[first_row[t_of_row]])
    np.testing.assert_array_equal(drs[:M], rs[first_row[t_of_row]])
    assert M < d["N"]


def test_reduce_order_hand_worked():
    """Level 2 adds in partition order from +0 in fp32: partials 1, 2^24, -2^24
    give ((0 + 1) + 2^24) - 2^24 = 0, because 2^24 + 1 rounds to 2^24 (tie to
    even); the reverse order would give 1."""
    T, H, P = 1, 8, 3
    vals = np.array([1.0, 2.0 ** 24, -(2.0 ** 24)], np.float32)
    part = np.repeat(to_bf16_bits(vals)[:, None], H, axis=1)
    tp_row = np.array([0, 1, 2], np.int32)
    out = oracle.combine_reduce(part, tp_row, T, H, P)
    assert np.all(out == 0)
    out_rev = oracle.combine_reduce(part[::-1].copy(), tp_row, T, H, P)   # rows reversed = order 2,1,0
    assert np.all(bf16_to_f32(out_rev) == 1.0)
