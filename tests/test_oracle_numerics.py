"""Pins of the oracle's fp8 (OCP E4M3 "fn") encoder and bf16 rounding.

Each check reaches the expected code another way than the oracle does:
hand-derived values, a nearest-value table search, torch's own casts.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import E4M3_VALUES, decode_e4m3fn, table_encode_e4m3fn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_points():
    pts = []
    with open(os.path.join(GOLDEN, "e4m3fn_points.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            v, code = line.split()[:2]
            pts.append((float(v), int(code, 16)))
    return pts


def test_golden_points_oracle_and_table():
    pts = _golden_points()
    assert len(pts) >= 25
    vals = np.array([p[0] for p in pts], np.float32)
    want = np.array([p[1] for p in pts], np.uint8)
    got = oracle.e4m3fn_encode(vals)
    np.testing.assert_array_equal(got, want)
    # the independent table encoder agrees with the hand-derived values too
    np.testing.assert_array_equal(table_encode_e4m3fn(vals), want)


def test_decode_matches_format_definition():
    for c in range(256):
        d = oracle.e4m3fn_decode(c)
        ref = decode_e4m3fn(c)
        if (c & 0x7F) == 0x7F:
            assert math.isnan(d) and np.isnan(ref)
        else:
            assert d == ref, hex(c)
    assert oracle.e4m3fn_decode(0x7E) == 448.0
    assert oracle.e4m3fn_decode(0x01) == 2.0 ** -9


def test_round_trip_all_finite_codes():
    # every representable value encodes to its own code
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]
    vals = decode_e4m3fn(codes).astype(np.float32)
    got = oracle.e4m3fn_encode(vals)
    np.testing.assert_array_equal(got, codes)


def _exhaustive_chunk(b0, b1):
    """First disagreement in fp32 bit patterns [b0, b1), or None."""
    bits = np.arange(b0, b1, dtype=np.uint32)
    v = bits.view(np.float32)
    got = oracle.e4m3fn_encode(v)
    ref = table_encode_e4m3fn(v)
    bad = np.nonzero(got != ref)[0]
    if bad.size:
        return ("table", hex(int(bits[bad[0]])), int(got[bad[0]]), int(ref[bad[0]]))
    m = np.abs(v) <= 464.0
    tv = torch.from_numpy(v[m]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(got[m] != tv)[0]
    if bad.size:
        return ("torch", hex(int(bits[m][bad[0]])), int(got[m][bad[0]]), int(tv[bad[0]]))
    return None


@pytest.mark.slow
def test_exhaustive_against_table_and_torch():
    """Every fp32 bit pattern with magnitude in [2^-12, 512): the oracle equals
    the nearest-value table encoder; where |v| <= 464 it also equals torch's
    float8_e4m3fn cast (which is round-to-nearest-even but not saturating).
    Chunks run on a few threads (the oracle call, numpy and torch release the
    GIL for the bulk of the work)."""
    import concurrent.futures
    lo = int(np.float32(2.0 ** -12).view(np.uint32))
    hi = int(np.float32(512.0).view(np.uint32))
    step = 1 << 23
    chunks = [(b0, min(b0 + step, hi)) for b0 in range(lo, hi, step)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        for res in ex.map(_exhaustive_chunk, *zip(*chunks)):
            assert res is None, res
    # below 2^-12 everything rounds to zero with its sign
    tiny = np.array([2.0 ** -13, 1e-20, 1e-45, 2.0 ** -126], np.float32)
    np.testing.assert_array_equal(oracle.e4m3fn_encode(tiny), np.zeros(4, np.uint8))
    np.testing.assert_array_equal(oracle.e4m3fn_encode(-tiny), np.full(4, 0x80, np.uint8))


def test_negative_mirror_and_random_patterns():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    got = oracle.e4m3fn_encode(v)
    ref = table_encode_e4m3fn(v)
    np.testing.assert_array_equal(got, ref)
    # sign symmetry
    fin = ~np.isnan(v)
    np.testing.assert_array_equal(oracle.e4m3fn_encode(-v[fin]), got[fin] ^ 0x80)


def test_max_element_of_block_encodes_to_448():
    """I9: for any amax > 0 in the normal range, amax / fp32(amax/448) encodes
    to 0x7E: the quotient is within an fp32 ulp or two of 448, and the E4M3
    neighbours of 448 are 416 and NaN."""
    rng = np.random.default_rng(3)
    amax = np.abs(rng.standard_normal(200_000).astype(np.float32)) * np.float32(8.0) + np.float32(1e-3)
    scale = (amax.astype(np.float64) / 448.0).astype(np.float32)
    q = (amax.astype(np.float64) / scale.astype(np.float64)).astype(np.float32)
    assert np.all(oracle.e4m3fn_encode(q) == 0x7E)


# ------------------------------------------------------------------------ bf16
def _torch_bf16(v):
    return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_rne_against_torch_random_patterns():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2 ** 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    # add the rounding neighbourhoods of every exponent: low halves 0x7FFF, 0x8000, 0x8001
    ex = (np.arange(0, 1 << 16, dtype=np.uint32) << 16)
    edge = np.concatenate([ex | 0x7FFF, ex | 0x8000, ex | 0x8001, ex | 0x0000, ex | 0xFFFF])
    bits = np.concatenate([bits, edge])
    v = bits.view(np.float32)
    fin = ~np.isnan(v)
    got = oracle.bf16_rne(v)
    np.testing.assert_array_equal(got[fin], _torch_bf16(v[fin]))
    # NaN stays NaN (exponent all ones, nonzero mantissa, quiet bit set), sign kept
    nanb = got[~fin]
    assert np.all((nanb & 0x7F80) == 0x7F80) and np.all((nanb & 0x0040) != 0)
    np.testing.assert_array_equal(nanb >> 15, (bits[~fin] >> 31).astype(np.uint16))


def test_bf16_rne_hand_values():
    cases = [
        (1.0, 0x3F80),
        (-2.0, 0xC000),
        (1.0 + 2.0 ** -8, 0x3F80),                 # midway 1 / 1+2^-7 -> even
        (1.0 + 3 * 2.0 ** -8, 0x3F82),             # midway -> even 0x3F82
        (3.3895313892515355e38, 0x7F7F),           # largest finite bf16 stays
        (3.4028234663852886e38, 0x7F80),           # largest fp32 rounds up past it -> inf
        (float("inf"), 0x7F80),
        (0.0, 0x0000),
        (-0.0, 0x8000),
    ]
    v = np.array([c[0] for c in cases], np.float32)
    np.testing.assert_array_equal(oracle.bf16_rne(v), np.array([c[1] for c in cases], np.uint16))


def test_e4m3_table_sanity():
    # independent closed-form facts about the value set
    assert E4M3_VALUES.size == 127
    assert E4M3_VALUES[1] == 2.0 ** -9 and E4M3_VALUES[8] == 2.0 ** -6
    assert E4M3_VALUES[0x38] == 1.0
