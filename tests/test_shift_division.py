"""The fused dedup kernel divides by multiply-shift: e / L as (e * m) >> 20
with m = floor(2^20 / L) + 1 for ids e < 1024 and L <= 1024, and p / K as
(p * m) >> 16 with m = floor(2^16 / K) + 1 for entries p < 4096 and K <= 16.
Checked exhaustively over those ranges in 32-bit unsigned arithmetic, as the
kernel computes it.  The counting kernel takes lane / K for lane < 16 as
trunc((lane + 1/2) * r) in fp32 with r the hardware reciprocal of K (within
1 ulp of 1/K): checked for every lane and K with r at the rounded reciprocal
and one ulp on either side."""
import numpy as np


def _check(a_max, d_max, s):
    a = np.arange(a_max, dtype=np.uint64)
    for d in range(1, d_max + 1):
        m = np.uint64((1 << s) // d + 1)
        prod = (a * m) & np.uint64(0xFFFFFFFF)          # the kernel's uint32 product
        assert np.all(a * m < (1 << 32)), d             # no wrap-around
        assert np.array_equal(prod >> np.uint64(s), a // np.uint64(d)), d


def test_expert_over_experts_per_partition():
    _check(1024, 1024, 20)


def test_entry_over_topk():
    _check(4096, 16, 16)


def test_lane_over_topk_by_reciprocal():
    lane = np.arange(16, dtype=np.float32)
    for k in range(1, 17):
        r0 = np.float32(1.0) / np.float32(k)
        for r in (np.nextafter(r0, np.float32(0)), r0, np.nextafter(r0, np.float32(1))):
            q = ((lane + np.float32(0.5)) * np.float32(r)).astype(np.float32)
            assert q.dtype == np.float32
            assert np.array_equal(np.trunc(q).astype(np.int64), np.arange(16) // k), (k, r)
