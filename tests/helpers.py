"""Independent checkers used to pin the oracle.

None of this calls the oracle or the HIP library: each helper is a second,
differently built way to reach the same definition (a nearest-value search
instead of exponent/mantissa rounding, exact rational arithmetic instead of
fmaf, a stable sort instead of a counting pass).
"""
from fractions import Fraction

import numpy as np

# ---------------------------------------------------------------- OCP E4M3 "fn"
# The 127 non-negative finite codes 0x00..0x7E (0x7F is NaN), valued from the
# format's definition: exponent field 0 -> m/8 * 2^-6, else (1 + m/8) * 2^(e-7).
_CODES = np.arange(0x7F, dtype=np.int64)
_EF, _MF = _CODES >> 3, _CODES & 7
E4M3_VALUES = np.where(_EF == 0, _MF / 8.0 * 2.0 ** -6,
                       (1.0 + _MF / 8.0) * np.exp2((_EF - 7).astype(np.float64)))
assert np.all(np.diff(E4M3_VALUES) > 0) and E4M3_VALUES[-1] == 448.0


def table_encode_e4m3fn(v32: np.ndarray) -> np.ndarray:
    """Nearest representable E4M3 value by search over the value table; ties go
    to the even code; |v| >= 448 saturates to 0x7E; NaN -> 0x7F; sign kept."""
    v = np.asarray(v32, dtype=np.float32)
    with np.errstate(invalid="ignore"):
        a = np.abs(v.astype(np.float64))
    sign = np.signbit(v).astype(np.uint8) << 7
    i = np.searchsorted(E4M3_VALUES, a)            # first value >= a
    hi = np.clip(i, 0, 126)
    lo = np.clip(i - 1, 0, 126)
    dlo = a - E4M3_VALUES[lo]
    dhi = E4M3_VALUES[hi] - a
    code = np.where(dhi < dlo, hi, lo)
    tie = (dhi == dlo) & (hi != lo)
    code = np.where(tie, np.where(hi % 2 == 0, hi, lo), code)
    code = np.where(a >= 448.0, 0x7E, code)
    code = np.where(np.isnan(a), 0x7F, code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def decode_e4m3fn(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    mag = c & 0x7F
    val = np.where(mag == 0x7F, np.nan, np.concatenate([E4M3_VALUES, [np.nan]])[mag])
    return np.where(c & 0x80, -val, val)


# ------------------------------------------------------------------ bf16 / fp32
def bf16_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def f32_bits(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def bf16_ordered(bits) -> np.ndarray:
    """Map bf16 bit patterns to integers whose difference counts ulps (+0 == -0)."""
    b = np.asarray(bits, dtype=np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def bf16_ulp_distance(a_bits, b_bits) -> np.ndarray:
    return np.abs(bf16_ordered(a_bits) - bf16_ordered(b_bits))


# --------------------------------------------------- exact rational fp32 rounding
def round_fraction_to_f32(q: Fraction) -> np.float32:
    """Round an exact rational to the nearest binary32 value, ties to even
    (normal and subnormal range; |q| below 2^128)."""
    if q == 0:
        return np.float32(0.0)
    s = -1 if q < 0 else 1
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    # now 2^e <= q < 2^(e+1)
    e = max(e, -126)                       # subnormals share the 2^-126 grid spacing
    scaled = q * Fraction(2) ** (23 - e)   # integer part = 24-bit significand
    m, rem = divmod(scaled.numerator, scaled.denominator)
    twice = 2 * rem
    if twice > scaled.denominator or (twice == scaled.denominator and (m & 1)):
        m += 1
    return np.float32(s * float(Fraction(m) * Fraction(2) ** (e - 23)))


def exact_fmaf(a, b, c) -> np.float32:
    return round_fraction_to_f32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


# ---------------------------------------------------------------- layout brute force
def brute_layout(idx: np.ndarray, E: int, P: int):
    """Rows by a stable sort of the valid (t,k) entries on expert id."""
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    n = flat.size
    valid = (flat >= 0) & (flat < E)
    vi = np.nonzero(valid)[0]
    order = vi[np.argsort(flat[vi], kind="stable")]
    row_of_pair = np.full(n, -1, np.int64)
    row_of_pair[order] = np.arange(order.size)
    src_pair = np.full(n, -1, np.int64)
    src_pair[:order.size] = order
    count = np.bincount(flat[vi], minlength=E)
    offset = np.concatenate([[0], np.cumsum(count)])
    L = E // P
    part_count = count.reshape(P, L).sum(axis=1)
    part_offset = np.concatenate([offset[0:E:L], [offset[E]]])
    status = 1 if np.any(flat >= E) else 0
    return dict(expert_count=count, expert_offset=offset, part_count=part_count,
                part_offset=part_offset, row_of_pair=row_of_pair, src_pair=src_pair,
                status=np.array([status]))


# ------------------------------------------------------- vectorised exact fmaf
def fmaf_exact_np(a, b, c) -> np.ndarray:
    """fp32 fma(a, b, c) with one rounding, vectorised: a*b is exact in fp64
    (24 + 24 bits), p + c is held exactly as a double-double (TwoSum), and the
    pair is rounded to fp32.  Rounding hi alone is correct unless hi is exactly
    an fp32 rounding midpoint, where the sign of lo decides."""
    a = np.asarray(a, np.float32).astype(np.float64)
    b = np.asarray(b, np.float32).astype(np.float64)
    c = np.asarray(c, np.float32).astype(np.float64)
    p = a * b
    hi = p + c
    bb = hi - p
    lo = (p - (hi - bb)) + (c - bb)
    r = hi.astype(np.float32)
    up = np.nextafter(r, np.float32(np.inf))
    dn = np.nextafter(r, np.float32(-np.inf))
    rd = r.astype(np.float64)
    mid_up = (rd + up.astype(np.float64)) * 0.5      # exact: fp32 neighbours fit in fp64
    mid_dn = (rd + dn.astype(np.float64)) * 0.5
    # hi sits on the midpoint above r (rounded down to even r) and lo > 0: round up
    r = np.where((hi == mid_up) & (lo > 0), up, r)
    # hi sits on the midpoint below r (rounded up to even r) and lo < 0: round down
    r = np.where((hi == mid_dn) & (lo < 0), dn, r)
    return r.astype(np.float32)
