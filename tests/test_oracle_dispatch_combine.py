"""Pins of the oracle's fp8 / bf16 dispatch and its combine.

Dispatch is rebuilt here from a different route: fp64 division rounded once
to fp32 (which equals IEEE fp32 division, 53 >= 2*24+2 bits) followed by the
nearest-value table encoder.  Combine is pinned bit-exactly by exact rational
fmaf on small cases, by an fp64 error bound at full size, and by the
identity-expert round trip (dispatch -> y = dequantised rows -> combine with
weights summing to 1 returns the dequantised input).
"""
import json
import os

import numpy as np
import pytest

import oracle
from tests.helpers import (bf16_to_f32, bf16_ulp_distance, decode_e4m3fn, exact_fmaf,
                           fmaf_exact_np, table_encode_e4m3fn)
from workloads import WORKLOADS, generate
from workloads.gen import to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def ref_quantise(x_bits):
    """Per token and 128-column block: scale = RN32(amax/448), q = enc(RN32(x/scale))."""
    x = bf16_to_f32(x_bits).astype(np.float64)
    T, H = x.shape
    xb = x.reshape(T, H // 128, 128)
    amax = np.max(np.abs(xb), axis=2)
    scale = (amax / 448.0).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (xb / scale.astype(np.float64)[..., None]).astype(np.float32)
    codes = table_encode_e4m3fn(q)
    codes[amax == 0] = 0
    return codes.reshape(T, H), scale


def test_hand_worked_block():
    g = json.load(open(os.path.join(GOLDEN, "dispatch_block.json")))
    x = np.full((1, 128), 1.0, np.float32)
    x[0, 0], x[0, 1] = 2.0, -1.0
    xb = to_bf16_bits(x)
    rop = np.array([0], np.int32)
    rx, rs = oracle.dispatch_fp8(xb, rop, 1)
    assert rs.view(np.uint32)[0, 0] == int(g["scale_bits"], 16)
    assert rx[0, 0] == int(g["codes"]["col0"], 16)
    assert rx[0, 1] == int(g["codes"]["col1"], 16)
    assert np.all(rx[0, 2:] == int(g["codes"]["default"], 16))


@pytest.mark.parametrize("name", ["tiny_4x1024", "ll_128x7168", "sweep_16x6144"])
def test_fp8_dispatch_against_fp64_route(name):
    wl = WORKLOADS[name]
    d = generate(wl, with_y=False)
    lo = oracle.layout(d["idx"], wl.E, wl.P)
    rx, rs = oracle.dispatch_fp8(d["x"], lo["row_of_pair"], wl.K)
    codes, scale = ref_quantise(d["x"])
    rop = lo["row_of_pair"].reshape(wl.T, wl.K)
    N = d["N"]
    for t in range(wl.T):
        for k in range(wl.K):
            r = rop[t, k]
            if r < 0:
                continue
            np.testing.assert_array_equal(rx[r], codes[t])              # I6: every copy identical
            np.testing.assert_array_equal(rs[r].view(np.uint32), scale[t].view(np.uint32))
    assert np.all(rx[N:] == 0) and np.all(rs[N:] == 0)                 # rows >= N untouched


def test_fp8_dispatch_zipf_slice_against_fp64_route():
    wl = WORKLOADS["bw_4096x7168_zipf"]
    d = generate(wl, with_y=False)
    lo = oracle.layout(d["idx"], wl.E, wl.P)
    t0, t1 = 1000, 1040
    rx, rs = oracle.dispatch_fp8(d["x"], lo["row_of_pair"], wl.K, t0=t0, t1=t1)
    codes, scale = ref_quantise(d["x"][t0:t1])
    rop = lo["row_of_pair"].reshape(wl.T, wl.K)
    for t in range(t0, t1):
        for r in rop[t]:
            np.testing.assert_array_equal(rx[r], codes[t - t0])
            np.testing.assert_array_equal(rs[r], scale[t - t0])


def test_dequantisation_bound_and_zero_block():
    """I7: |dec(q)*scale - x| <= 2^-4 |x| + 2^-10 scale (+ fp32 slack); amax = 0
    gives scale 0 and zero bytes."""
    wl = WORKLOADS["ll_128x7168"]
    d = generate(wl, with_y=False)
    x = d["x"].copy()
    x[3, 256:384] = 0                        # one all-zero block
    x[5, 128:256] = 0x8000                   # a block of -0.0
    rop = np.arange(wl.T, dtype=np.int32)    # K = 1, identity rows
    rx, rs = oracle.dispatch_fp8(x, rop, 1)
    assert rs[3, 2] == 0 and np.all(rx[3, 256:384] == 0)
    assert rs[5, 1] == 0 and np.all(rx[5, 128:256] == 0)
    xf = bf16_to_f32(x).astype(np.float64)
    sc = np.repeat(rs.astype(np.float64), 128, axis=1)
    deq = decode_e4m3fn(rx) * sc
    err = np.abs(deq - xf)
    bound = 2.0 ** -4 * np.abs(xf) + 2.0 ** -10 * sc + 1e-6 * np.abs(xf)
    assert np.all(err <= bound)
    # the outlier row's blocks carry ~50x scales
    row = d["meta"]["outlier_rows"][0]
    assert np.median(rs[row]) > 20 * np.median(rs)


def test_bf16_passthrough_copies_rows():
    wl = WORKLOADS["masked_16384x4096_bf16"].with_(T=64)
    d = generate(wl, with_y=False)
    lo = oracle.layout(d["idx"], wl.E, wl.P)
    rx = oracle.dispatch_bf16(d["x"], lo["row_of_pair"], wl.K)
    src = lo["src_pair"]
    N = d["N"]
    np.testing.assert_array_equal(rx[:N], d["x"][src[:N] // wl.K])
    assert np.all(rx[N:] == 0)


# ------------------------------------------------------------------- combine
def test_combine_exact_rational_small():
    """Bit-exact pin: acc = fmaf(w, y, acc) in k order from +0, masked entries
    skipped, then bf16 round-to-nearest-even -- with fmaf done in exact
    rational arithmetic and one rounding per step."""
    rng = np.random.default_rng(99)
    T, H, K, E, P = 5, 16, 6, 12, 3
    idx = rng.integers(-1, E, size=(T, K)).astype(np.int32)
    idx[4] = -1                                          # an all-masked token
    w = rng.standard_normal((T, K)).astype(np.float32)
    lo = oracle.layout(idx, E, P)
    y = to_bf16_bits(rng.standard_normal((T * K, H)).astype(np.float32) * 3)
    got = oracle.combine(y, lo["row_of_pair"], w, T, H, K)
    rop = lo["row_of_pair"].reshape(T, K)
    yf = bf16_to_f32(y)
    for t in range(T):
        for c in range(H):
            acc = np.float32(0.0)
            for k in range(K):
                r = rop[t, k]
                if r >= 0:
                    acc = exact_fmaf(w[t, k], yf[r, c], acc)
            want = to_bf16_bits(np.array([acc], np.float32))[0]
            assert got[t, c] == want, (t, c)
    assert np.all(got[4] == 0)                            # all masked -> +0


def test_vectorised_fmaf_matches_exact_rationals():
    """The numpy fmaf used below, against exact rational arithmetic, on random
    operands and on operands built to land on fp32 rounding midpoints."""
    rng = np.random.default_rng(17)
    a = rng.standard_normal(3000).astype(np.float32)
    b = rng.standard_normal(3000).astype(np.float32)
    c = rng.standard_normal(3000).astype(np.float32) * np.float32(4.0)
    # midpoint cases: a*b exactly half an ulp of c plus/minus a tiny excess
    c2 = np.float32(1.0) + np.arange(1, 1001, dtype=np.float32) * np.float32(2.0 ** -20)
    a2 = np.full(1000, 2.0 ** -24, np.float32)
    b2 = np.where(np.arange(1000) % 3 == 0, 1.0, np.where(np.arange(1000) % 3 == 1, 1.0 + 2.0 ** -23,
                                                          1.0 - 2.0 ** -24)).astype(np.float32)
    a, b, c = np.concatenate([a, a2, -a2]), np.concatenate([b, b2, b2]), np.concatenate([c, c2, c2])
    got = fmaf_exact_np(a, b, c)
    for i in range(a.size):
        assert got[i] == exact_fmaf(a[i], b[i], c[i]), i


@pytest.mark.parametrize("name", ["ll_128x7168", "tiny_4x1024"])
def test_combine_bit_exact_at_full_size(name):
    """Bit-exact pin at full size: the fmaf chain in k order from +0 (masked
    entries skipped), evaluated with the vectorised exact fmaf, then torch's
    bf16 rounding."""
    wl = WORKLOADS[name]
    d = generate(wl)
    lo = oracle.layout(d["idx"], wl.E, wl.P)
    got = oracle.combine(d["y"], lo["row_of_pair"], d["w"], wl.T, wl.H, wl.K)
    rop = lo["row_of_pair"].reshape(wl.T, wl.K)
    yf = bf16_to_f32(d["y"])
    acc = np.zeros((wl.T, wl.H), np.float32)
    for k in range(wl.K):
        r = rop[:, k]
        valid = r >= 0
        upd = fmaf_exact_np(np.broadcast_to(d["w"][:, k:k + 1], acc.shape), yf[np.maximum(r, 0)], acc)
        acc = np.where(valid[:, None], upd, acc)
    np.testing.assert_array_equal(got, to_bf16_bits(acc))


def test_combine_fp64_bound_full_size():
    wl = WORKLOADS["ll_128x7168"]
    d = generate(wl)
    lo = oracle.layout(d["idx"], wl.E, wl.P)
    got = oracle.combine(d["y"], lo["row_of_pair"], d["w"], wl.T, wl.H, wl.K)
    rop = lo["row_of_pair"].reshape(wl.T, wl.K)
    yf = bf16_to_f32(d["y"]).astype(np.float64)
    w = d["w"].astype(np.float64)
    exact = np.zeros((wl.T, wl.H))
    mag = np.zeros((wl.T, wl.H))
    for k in range(wl.K):
        r = rop[:, k]
        exact += w[:, k:k + 1] * yf[r]
        mag += np.abs(w[:, k:k + 1] * yf[r])
    g = bf16_to_f32(got).astype(np.float64)
    # K fp32 roundings (each <= 2^-24 of the running magnitude) + one bf16 rounding
    bound = wl.K * 2.0 ** -24 * mag + 2.0 ** -8 * np.abs(exact) + 1e-38
    assert np.all(np.abs(g - exact) <= bound)


def test_identity_experts_return_dequantised_input():
    """I5: y = bf16(dequantised row), weights summing to 1 -> combine returns the
    dequantised input within 1 bf16 ulp."""
    wl = WORKLOADS["tiny_4x1024"]
    d = generate(wl, with_y=False)
    lo = oracle.layout(d["idx"], wl.E, wl.P)
    rx, rs = oracle.dispatch_fp8(d["x"], lo["row_of_pair"], wl.K)
    N = d["N"]
    deq = (decode_e4m3fn(rx[:N]) * np.repeat(rs[:N].astype(np.float64), 128, axis=1)).astype(np.float32)
    y = np.zeros((wl.T * wl.K, wl.H), np.uint16)
    y[:N] = to_bf16_bits(deq)
    out = oracle.combine(y, lo["row_of_pair"], d["w"], wl.T, wl.H, wl.K)
    codes, scale = ref_quantise(d["x"])
    deq_x = to_bf16_bits((decode_e4m3fn(codes) * np.repeat(scale.astype(np.float64), 128, axis=1)).astype(np.float32))
    assert np.max(bf16_ulp_distance(out, deq_x)) <= 1
    assert abs(float(d["w"].sum(axis=1).max()) - 1.0) < 1e-6


def test_k1_unit_weight_returns_y_and_bf16_identity():
    """I10: K = 1, w = 1 returns y exactly; I8: bf16 passthrough + identity
    experts + unit-sum weights returns x within 1 ulp."""
    rng = np.random.default_rng(4)
    T, H = 7, 256
    idx = rng.integers(0, 8, size=(T, 1)).astype(np.int32)
    lo = oracle.layout(idx, 8, 2)
    y = to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    out = oracle.combine(y, lo["row_of_pair"], np.ones((T, 1), np.float32), T, H, 1)
    src = lo["src_pair"]
    np.testing.assert_array_equal(out[src // 1], y)

    wl = WORKLOADS["masked_16384x4096_bf16"].with_(T=32, H=512)
    d = generate(wl, with_y=False)
    lo = oracle.layout(d["idx"], wl.E, wl.P)
    rx = oracle.dispatch_bf16(d["x"], lo["row_of_pair"], wl.K)
    out = oracle.combine(rx, lo["row_of_pair"], d["w"], wl.T, wl.H, wl.K)
    has = (d["idx"] >= 0).any(axis=1)
    assert np.max(bf16_ulp_distance(out[has], d["x"][has])) <= 1
