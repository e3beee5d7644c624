"""GPU parity of the per-destination (dedup) path against the oracle.

ep_dedup_layout, the dedup dispatch (ep_dispatch with K = P over tp_row),
ep_combine_partial and ep_combine_reduce, each output compared with the
oracle: layout and fp8/scales/bf16 rows bit-exact, partial and output rows
within 1 bf16 ulp (and in practice bit-exact: the same fmaf order and the
same partition-order fp32 adds).
"""
import numpy as np
import pytest

from tests.pathrun import compare_dedup, run_gpu_dedup, run_oracle_dedup
from workloads import WORKLOADS, generate

pytestmark = pytest.mark.gpu


def _case(wl, seed=None, d=None, fused=False, geometry=None):
    print("dedup case %s T=%d H=%d E=%d P=%d K=%d %s seed=%s fused=%s geometry=%s" % (
        wl.name, wl.T, wl.H, wl.E, wl.P, wl.K, wl.payload, seed, fused, geometry), flush=True)
    d = generate(wl, seed=seed) if d is None else d
    got = run_gpu_dedup(wl, d, fused=fused, geometry=geometry)
    ref = run_oracle_dedup(wl, d)
    ndiff = compare_dedup(wl, got, ref)
    assert ndiff == 0, "%s: %d partial/output values differ by 1 ulp" % (wl.name, ndiff)
    return got, ref, d


@pytest.mark.parametrize("name", ["tiny_4x1024", "ll_128x7168", "sweep_4x6144", "sweep_16x6144",
                                  "bw_4096x7168_zipf", "masked_16384x4096_bf16"])
def test_dedup_workloads(name):
    wl = WORKLOADS[name]
    _case(wl, wl.seed + 11)


def test_dedup_few_partitions_many_shared():
    """E = 32, P = 8, K = 8: most tokens reach a partition through several of
    their experts (kmask with several bits)."""
    wl = WORKLOADS["ll_128x7168"].with_(name="dedup_e32_p8", E=32, P=8)
    got, ref, _ = _case(wl, 21)
    km = ref["kmask"]
    assert np.count_nonzero([bin(int(v)).count("1") > 1 for v in km]) > wl.T


def test_dedup_reduce_both_copy_regimes():
    """ep_combine_reduce compacts the present copies of a token with at most 8
    of them and loops over the partitions above that: top-16 over 16
    partitions of 4 experts, 30 % of entries masked, gives tokens of both
    kinds (6 to 12 copies) in one launch."""
    wl = WORKLOADS["ll_128x7168"].with_(name="dedup_k16_p16_copies", T=96, H=1536, K=16, E=64,
                                        P=16, mask_frac=0.3)
    got, ref, _ = _case(wl, 33)
    copies = (np.asarray(ref["tp_row"]).reshape(wl.T, wl.P) >= 0).sum(axis=1)
    assert (copies > 8).any() and (copies <= 8).any()


DEDUP_EDGE = {
    "T1": dict(T=1),
    "P1": dict(P=1, E=32),
    "K1": dict(K=1),
    "K16_P16": dict(K=16, E=64, P=16),
    "H640": dict(H=640, T=33),
    "T256_P8": dict(T=256, H=256, P=8),                  # ep_dedup_layout: one thread per token
    "T512_P8": dict(T=512, H=256, P=8),
    "T513_P8": dict(T=513, H=256, P=8),
    "token_kernel_limit_1024": dict(T=1024, H=128, E=64, P=16),   # 16 waves, every partition
    "over_token_kernel_1025": dict(T=1025, H=128, P=8),  # T*P = 8200: chunked couples
    "single_wg_P1_T2000": dict(T=2000, H=128, E=32, P=1),  # T*P = 2000: single-workgroup couples
    "many_chunks_scan_pass": dict(T=40000, H=128, E=64, P=8),   # > 256 chunks of couples
    "bf16": dict(payload="bf16", T=50, H=512),
}


@pytest.mark.parametrize("edge", list(DEDUP_EDGE))
def test_dedup_edge_shapes(edge):
    wl = WORKLOADS["tiny_4x1024"].with_(name="dedup_" + edge, **DEDUP_EDGE[edge])
    _case(wl, 79)


FUSED_NAMES = ["tiny_4x1024", "ll_128x7168", "sweep_4x6144", "sweep_8x6144", "sweep_16x6144",
               "bw_4096x7168_zipf"]


@pytest.mark.parametrize("name", FUSED_NAMES)
def test_dedup_layout_dispatch(name):
    """ep_dedup_layout_dispatch (one launch up to T*K = 2048, three kernels
    above): both layouts, dedup rows and scales equal to the oracle."""
    wl = WORKLOADS[name]
    _case(wl, wl.seed + 12, fused=True)


FUSED_EDGE = {
    "T1": dict(T=1),
    "P1": dict(P=1, E=32),
    "K1_many_tokens": dict(K=1, T=2048, H=128),          # 2048 tokens, one per lane of 8 waves
    "K16_P16": dict(K=16, E=64, P=16),
    "E1024_P16": dict(E=1024, P=16, T=64),               # L = 64
    "E1024_P1": dict(E=1024, P=1, T=40),                 # L = 1024: the shift divide at its limit
    "E96_P3": dict(E=96, P=3, T=50),                     # P not a power of two
    "H128_tokens_share_wg": dict(H=128, T=200),          # 4 tokens per workgroup
    "H640": dict(H=640, T=33),
    "at_limit_2048": dict(T=256, H=256),
    "over_limit_2056": dict(T=257, H=256),
    "at_limit_4096": dict(T=512, H=256),
    "over_limit_4104": dict(T=513, H=256),
    "w8_4096_ids": dict(T=300, H=7168, E=32, P=8),
    "bf16": dict(payload="bf16", T=50, H=512),
    "w8_K16_T128": dict(T=128, K=16, E=64, P=16, H=7168),
    "w8_two_steps": dict(T=1024, K=2, H=1024),
    # T*K <= 1024, K a power of two, 8/7/6 waves dividing the steps per token:
    # the counting kernel (one token per workgroup)
    "count_T1": dict(T=1, H=7168),
    "count_w7_P1": dict(T=100, H=7168, E=32, P=1),
    "count_w6_K16_P16": dict(T=64, K=16, E=64, P=16, H=6144),
    "count_w8_K4": dict(T=256, K=4, E=64, P=8, H=4096),
    "count_w6_K1": dict(T=500, K=1, E=32, P=4, H=3072),
    "count_w7_K2_E1024_P16": dict(T=300, K=2, E=1024, P=16, H=3584),
    "count_E1024_P1": dict(T=40, E=1024, P=1, H=3584),
    "count_P3": dict(T=100, E=96, P=3, H=7168),
    "count_ragged_H6016": dict(T=60, H=6016),         # 12 steps, the last one 384 columns
    "count_bf16": dict(payload="bf16", T=64, H=6144),
}


@pytest.mark.parametrize("edge", list(FUSED_EDGE))
def test_dedup_layout_dispatch_edges(edge):
    wl = WORKLOADS["tiny_4x1024"].with_(name="dedup_fused_" + edge, **FUSED_EDGE[edge])
    _case(wl, 80, fused=True)


@pytest.mark.parametrize("K,H", [(6, 256), (8, 3584)])    # general kernel; counting kernel
def test_dedup_fused_masked_duplicate_and_bad_ids(K, H):
    wl = WORKLOADS["tiny_4x1024"].with_(name="dedup_fused_ids", T=40, H=H, E=16, P=4, K=K)
    d = generate(wl, seed=9)
    rng = np.random.default_rng(9)
    idx = rng.integers(-3, 20, size=(wl.T, wl.K)).astype(np.int32)
    idx[3] = 7
    idx[4] = -1
    idx[5] = 99
    d["idx"] = idx
    got, ref, _ = _case(wl, d=d, fused=True)
    assert int(got["status"][0]) == 1


@pytest.mark.parametrize("T", [40, 20])      # 160 couples; 80: the one-wave layout
def test_dedup_masked_duplicate_and_bad_ids(T):
    wl = WORKLOADS["tiny_4x1024"].with_(name="dedup_ids", T=T, H=256, E=16, P=4, K=6)
    d = generate(wl, seed=8)
    rng = np.random.default_rng(8)
    idx = rng.integers(-3, 20, size=(wl.T, wl.K)).astype(np.int32)
    idx[3] = 7            # every entry on one expert: one couple, all six bits
    idx[4] = -1           # nothing present: output +0
    idx[5] = 99           # only bad ids
    d["idx"] = idx
    got, ref, _ = _case(wl, d=d)
    assert int(got["status"][0]) == 1
    assert np.all(got["out"][4] == 0) and np.all(got["out"][5] == 0)
    assert int(got["kmask"][3 * wl.P + 7 // (wl.E // wl.P)]) == 0x3F


@pytest.mark.parametrize("fused", [False, True])
def test_dedup_empty_batch(fused):
    """T = 0 through ep_dedup_layout, and through ep_dedup_layout_dispatch
    (the plain layout's outputs included): zero counts and offsets, clean
    status."""
    import torch
    import combine_ep_layout_05_amd as ep
    print("dedup case T=0 fused=%s" % fused, flush=True)
    db = ep.EpDedupBuffers(0, 1024, 8, 32, 8)
    idx = torch.empty((0, 8), dtype=torch.int32, device="cuda")
    for t in (db.part_tokens, db.part_token_offset, db.status):
        t.fill_(-7)
    if fused:
        # the per-expert layout goes to `buf`, the status (one for the call) to db
        buf = ep.EpBuffers(0, 1024, 8, 32, 8)
        for t in (buf.expert_count, buf.expert_offset, buf.part_count, buf.part_offset):
            t.fill_(-7)
        db.layout_dispatch(idx, torch.empty((0, 1024), dtype=torch.bfloat16, device="cuda"), buf)
        torch.cuda.synchronize()
        for t in (buf.expert_count, buf.expert_offset, buf.part_count, buf.part_offset):
            assert np.all(t.cpu().numpy() == 0)
    else:
        db.layout(idx)
    torch.cuda.synchronize()
    assert np.all(db.part_tokens.cpu().numpy() == 0)
    assert np.all(db.part_token_offset.cpu().numpy() == 0)
    assert int(db.status.cpu()[0]) == 0


@pytest.mark.parametrize("overlap", [False, True])
def test_combine_partial_hand_built_masks(overlap):
    """ep_combine_partial on masks built by hand rather than by the dedup
    layout: present couples with several entries, a single entry, no entry,
    or only entries whose receive row is -1 (each gets +0), bits at or above
    K (ignored), and -- with overlap=True -- an entry in two partitions' masks
    for some tokens (summed into both).  Partial rows of present couples
    bit-exact against the oracle, absent couples' rows untouched; then the
    reduce on the same couples."""
    import torch
    import combine_ep_layout_05_amd as ep
    import oracle
    from tests.pathrun import to_dev
    T, H, K, P = 53, 1536, 8, 6
    rng = np.random.default_rng(977 + overlap)
    n = T * K
    rop = rng.permutation(n).astype(np.int32)
    rop[rng.random(n) < 0.1] = -1
    y = (rng.standard_normal((n, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    w = rng.random((T, K)).astype(np.float32)
    present = rng.random((T, P)) < 0.6
    tp_row = np.full((T, P), -1, np.int32)
    tp_row[present] = rng.permutation(int(present.sum())).astype(np.int32)
    kmask = np.zeros((T, P), np.uint32)
    for t in range(T):
        ps = np.nonzero(present[t])[0]
        if ps.size == 0:
            continue
        owner = rng.choice(ps, size=K)                  # each entry in one present partition
        for k in range(K):
            kmask[t, owner[k]] |= np.uint32(1 << k)
        if t % 5 == 0:
            kmask[t, ps[0]] = 0                         # a present couple with no entry
        if t % 7 == 1:
            kmask[t, ps[-1]] |= np.uint32(1 << K)       # a bit above K: ignored
        if overlap and t % 3 == 0 and ps.size > 1:
            kmask[t, ps[1]] |= kmask[t, ps[0]] | np.uint32(1)   # entries in two masks
    M = int(present.sum())
    ref = oracle.combine_partial(y, rop, w, tp_row, kmask, T, H, K, P, rows=T * P)
    part = torch.full((T * P, H), 0x5A5A, dtype=torch.int16, device="cuda")
    ep.ep_combine_partial(to_dev(y.view(np.int16), torch.bfloat16), to_dev(rop), to_dev(w),
                          to_dev(tp_row.reshape(-1)), to_dev(kmask.reshape(-1).view(np.int32)), P,
                          part)
    torch.cuda.synchronize()
    got = part.cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got[:M], ref[:M])
    assert np.all(got[M:] == 0x5A5A)
    out = torch.full((T, H), 0x5A5A, dtype=torch.int16, device="cuda")
    ep.ep_combine_reduce(part, to_dev(tp_row.reshape(-1)), T, P, out)
    torch.cuda.synchronize()
    want = oracle.combine_reduce(ref, tp_row, T, H, P)
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint16), want)


@pytest.mark.parametrize("fused", [False, True])
def test_dedup_masked_entries_never_use_row0(fused):
    """The partial combine reads row 0 of the expert outputs for the slots past
    a token's entries (an in-bounds stand-in) and never stores what they add:
    with row 0 at +inf and a quarter of the entries masked, partials and
    outputs still equal the oracle's."""
    wl = WORKLOADS["tiny_4x1024"].with_(name="dedup_row0_inf", T=40, H=1024, E=64, P=8, K=8)
    d = generate(wl, seed=32)
    rng = np.random.default_rng(32)
    idx = d["idx"].copy()
    idx[rng.random(idx.shape) < 0.25] = -1
    d["idx"] = idx
    y = d["y"].copy()
    y[0, :] = 0x7F80                                    # bf16 +inf
    d["y"] = y
    _case(wl, d=d, fused=fused)


# ep_dedup_layout_dispatch_geom: every workgroup size the fused dedup kernels
# take, and dispatch geometries of the unfused path, against the oracle.
# (shape, geometry, kernel the plan must report)
DEDUP_GEOMETRY = {
    "count_w8_24steps": (dict(T=64, H=12288, E=256, P=8), (8, 0, 0), "fused_count"),
    "count_w6_24steps": (dict(T=64, H=12288, E=256, P=8), (6, 0, 0), "fused_count"),
    "general_w4_24steps": (dict(T=64, H=12288, E=256, P=8), (4, 0, 0), "fused_general"),
    "count_w7_14steps": (dict(T=128, H=7168, E=288, P=16), (7, 0, 0), "fused_count"),
    "general_w8_14steps": (dict(T=128, H=7168, E=288, P=16), (8, 0, 0), "fused_general"),
    "general_w4_14steps": (dict(T=128, H=7168, E=288, P=16), (4, 0, 0), "fused_general"),
    "general_w8_2048": (dict(T=256, H=1536, E=64, P=8), (8, 0, 0), "fused_general"),
    "general_w4_2048_bf16": (dict(T=256, H=1536, E=64, P=8, payload="bf16"), (4, 0, 0),
                             "fused_general"),
    "unfused_w1": (dict(T=640, H=1536, E=64, P=8), (1, 0, 512), "layout_then_dispatch"),
    "unfused_w2_cap_slice1024": (dict(T=640, H=1536, E=64, P=8), (2, 256, 1024),
                                 "layout_then_dispatch"),
    "unfused_w8_cap64_slice1024_bf16": (dict(T=640, H=1536, E=64, P=8, payload="bf16"),
                                        (8, 64, 1024), "layout_then_dispatch"),
    # the shipped rule's geometry for 16384 x 4096 bf16, on a smaller batch
    "unfused_w1_cap1024_bf16": (dict(T=640, H=4096, E=128, P=8, payload="bf16"), (1, 1024, 512),
                                "layout_then_dispatch"),
}


@pytest.mark.parametrize("case", sorted(DEDUP_GEOMETRY))
def test_dedup_layout_dispatch_geometry(case):
    import combine_ep_layout_05_amd as ep
    shape, geometry, kernel = DEDUP_GEOMETRY[case]
    wl = WORKLOADS["ll_128x7168"].with_(name="dedup_geom_" + case, **shape)
    plan = ep.ep_dedup_layout_dispatch_plan(wl.T, wl.H, wl.K, wl.E, wl.P, wl.payload, geometry)
    assert plan["kernel"] == kernel and plan["waves"] == geometry[0], plan
    _case(wl, 60 + len(case), fused=True, geometry=geometry)
