"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar (the method's own contract): layout outputs, fp8 bytes, fp32 scales and
bf16 passthrough rows bit-exact; combine within 1 bf16 ulp (relative error
<= 2^-7 = 7.8e-3), and in practice bit-exact because both sides use fmaf in
the same k order.  Rows past N must stay untouched (receive buffers are
poisoned first).
"""
import sys

import numpy as np
import pytest

from tests.helpers import bf16_to_f32
from tests.pathrun import compare, run_gpu, run_oracle
from workloads import WORKLOADS, generate

pytestmark = pytest.mark.gpu

SMALL = ["tiny_4x1024", "ll_128x7168", "sweep_4x6144", "sweep_8x6144", "sweep_16x6144"]
LARGE = ["bw_4096x7168_zipf", "masked_16384x4096_bf16"]


def _case(wl, seed=None, d=None, fused=False):
    print("case %s T=%d H=%d E=%d P=%d K=%d %s seed=%s fused=%s" % (
        wl.name, wl.T, wl.H, wl.E, wl.P, wl.K, wl.payload, seed, fused), flush=True)
    sys.stdout.flush()
    d = generate(wl, seed=seed) if d is None else d
    got = run_gpu(wl, d, fused=fused)
    ref = run_oracle(wl, d)
    ndiff = compare(wl, got, ref)
    assert ndiff == 0, "%s: %d combine outputs differ by 1 ulp" % (wl.name, ndiff)
    return got, ref, d


@pytest.mark.parametrize("name", SMALL)
@pytest.mark.parametrize("dseed", [0, 100, 200])
def test_small_workloads(name, dseed):
    wl = WORKLOADS[name]
    _case(wl, wl.seed + dseed)


@pytest.mark.parametrize("name", LARGE)
def test_large_workloads(name):
    wl = WORKLOADS[name]
    _case(wl, wl.seed)


BENCH_WORKLOADS = ["ll_128x7168", "sweep_4x6144", "sweep_8x6144", "sweep_16x6144",
                   "bw_4096x7168_zipf", "masked_16384x4096_bf16"]


@pytest.mark.parametrize("name", BENCH_WORKLOADS)
def test_bench_launch_configuration(name):
    """Every workload bench.py times, in the launch configuration it times:
    ep_layout_dispatch then ep_combine with the saved tuned geometry, at full
    size, against the oracle."""
    import bench
    wl = WORKLOADS[name]
    d = generate(wl, seed=wl.seed)
    print("bench configuration %s (geometry %s)" % (name, bench.GEOMETRY), flush=True)
    got = run_gpu(wl, d, fused=True, geometry=bench.GEOMETRY)
    ref = run_oracle(wl, d)
    assert compare(wl, got, ref) == 0


@pytest.mark.parametrize("name", SMALL + LARGE)
def test_fused_layout_dispatch(name):
    """ep_layout_dispatch: one launch up to 2048 entries, layout + dispatch
    kernels above; same results as the separate calls, hence as the oracle."""
    wl = WORKLOADS[name]
    _case(wl, wl.seed + 1, fused=True)


FUSED_EDGE = {
    "T1": dict(T=1),
    "K16": dict(K=16, E=64, P=8),
    "E1024": dict(E=1024, P=8, T=64),
    "H128_many_tokens_per_wg": dict(H=128, T=200),        # 1 step/token: 4 tokens per workgroup
    "H640": dict(H=640, T=33),
    "at_2048": dict(T=256, H=256),                        # T*K = 2048: the 2048-id instance
    "over_2048": dict(T=257, H=256),                      # T*K = 2056: the 4096-id instance
    "at_limit_4096": dict(T=512, H=256),                  # T*K = 4096: fused
    "over_limit_4104": dict(T=513, H=256),                # T*K = 4104: layout + dispatch
    "w8_4096_ids": dict(T=300, H=7168),                   # 4096-id instance with 8-wave workgroups
    "bf16_payload": dict(payload="bf16", T=50, H=512),
    # more than 1024 items: 8-wave workgroups
    "w8_K16_T128": dict(T=128, K=16, E=64, P=8, H=7168),
    "w8_one_step_8_tokens_per_wg": dict(T=2048, K=1, H=128),
    "w8_two_steps": dict(T=1024, K=2, H=1024),
    "w8_bf16_ragged": dict(payload="bf16", T=200, H=5000 // 8 * 8 + 8),
    # at most 128 entries: the barrier-free kernel (every wave ranks its own token)
    "tiny_n1": dict(T=1, K=1),
    "tiny_n64_one_round": dict(T=8),
    "tiny_n65_two_rounds_odd_K": dict(T=13, K=5, E=40, P=8),
    "tiny_n128_K16": dict(T=8, K=16, E=64, P=8),
    "tiny_E1024": dict(T=4, E=1024, P=8),
    "tiny_bf16": dict(payload="bf16", T=4, H=1024),
    "tiny_K3_one_step_tokens": dict(T=40, K=3, H=128),
    "general_n136": dict(T=17),
    # 128 < T*K <= 1024: the counting kernel (workgroups of 8, 7 or 6 waves)
    "count_w7_half_token": dict(T=100, H=7168),
    "count_w6": dict(T=64, H=6144),
    "count_w8_two_tokens": dict(T=120, H=2048),
    "count_w8_straddling_11_steps": dict(T=90, H=5632),
    "count_bf16": dict(payload="bf16", T=64, H=7168),
    "count_K3_w6_two_tokens": dict(T=300, K=3, H=1536),
    "count_E1024": dict(T=100, E=1024, P=8, H=7168),
    "general_just_over_1024": dict(T=129, H=7168),
}


@pytest.mark.parametrize("edge", list(FUSED_EDGE))
def test_fused_edge_shapes(edge):
    wl = WORKLOADS["tiny_4x1024"].with_(name="fused_" + edge, **FUSED_EDGE[edge])
    _case(wl, 78, fused=True)


def test_fused_masked_duplicate_and_bad_ids():
    wl = WORKLOADS["tiny_4x1024"].with_(name="fused_ids", T=40, H=256, E=16, P=4, K=6)
    d = generate(wl, seed=6)
    rng = np.random.default_rng(6)
    idx = rng.integers(-3, 20, size=(wl.T, wl.K)).astype(np.int32)
    idx[3] = 7
    idx[4] = -1
    d["idx"] = idx
    got, ref, _ = _case(wl, d=d, fused=True)
    assert int(got["status"][0]) == 1


def test_fused_count_masked_duplicate_and_bad_ids():
    """The counting kernel (128 < T*K <= 1024) on masked, repeated and
    out-of-range ids."""
    wl = WORKLOADS["tiny_4x1024"].with_(name="fused_count_ids", T=100, H=7168, E=16, P=4, K=6)
    d = generate(wl, seed=26)
    rng = np.random.default_rng(26)
    idx = rng.integers(-3, 20, size=(wl.T, wl.K)).astype(np.int32)
    idx[3] = 7
    idx[4] = -1
    d["idx"] = idx
    got, ref, _ = _case(wl, d=d, fused=True)
    assert int(got["status"][0]) == 1


def test_fused_tiny_masked_duplicate_and_bad_ids():
    """The barrier-free kernel (T*K <= 128) on masked, repeated and
    out-of-range ids."""
    wl = WORKLOADS["tiny_4x1024"].with_(name="fused_tiny_ids", T=20, H=256, E=16, P=4, K=6)
    d = generate(wl, seed=16)
    rng = np.random.default_rng(16)
    idx = rng.integers(-3, 20, size=(wl.T, wl.K)).astype(np.int32)
    idx[3] = 7
    idx[4] = -1
    d["idx"] = idx
    got, ref, _ = _case(wl, d=d, fused=True)
    assert int(got["status"][0]) == 1


EDGE = {
    "T1": dict(T=1),
    "K1": dict(K=1),
    "K16": dict(K=16, E=64, P=8),
    "E_eq_P": dict(E=16, P=16, K=4),
    "H128": dict(H=128),
    "H640_ragged_step": dict(H=640),
    "H1152": dict(H=1152),
    "E1024": dict(E=1024, P=8, T=64),
    "count_layout_n136": dict(T=17, H=256),           # ep_layout by ballot counting, ragged 8
    "count_layout_n1024_E1024": dict(T=128, H=256, E=1024, P=16),
    "count_layout_n1032": dict(T=129, H=256),         # two ids per thread
    "single_wg_limit": dict(T=256, H=256),            # 2048 pairs: the counting layout at its limit
    "just_over_single_wg": dict(T=257, H=256),        # 2056 pairs -> chunked path, ragged chunk
    "chunked_4104": dict(T=513, H=256),
    "chunked_ragged": dict(T=700, H=384, E=96, P=4),
    "many_chunks_scan_pass": dict(T=70000, H=128, E=64, P=8),   # > 256 chunks: scan launch
}


@pytest.mark.parametrize("edge", list(EDGE))
def test_edge_shapes(edge):
    wl = WORKLOADS["tiny_4x1024"].with_(name="edge_" + edge, **EDGE[edge])
    _case(wl, 77)


@pytest.mark.parametrize("T", [40, 20])      # 240 entries; 120: the one-wave layout
def test_masked_duplicate_and_bad_ids(T):
    wl = WORKLOADS["tiny_4x1024"].with_(name="edge_ids", T=T, H=256, E=16, P=4, K=6)
    d = generate(wl, seed=5)
    rng = np.random.default_rng(5)
    idx = rng.integers(-3, 20, size=(wl.T, wl.K)).astype(np.int32)   # masks, bad ids >= 16
    idx[3] = 7                                                        # all-duplicate token
    idx[4] = -1                                                       # all-masked token
    d["idx"] = idx
    got, ref, _ = _case(wl, d=d)
    assert int(got["status"][0]) == 1
    assert np.all(got["out"][4] == 0)


def test_all_masked_batch():
    wl = WORKLOADS["tiny_4x1024"].with_(name="edge_all_masked", T=9)
    d = generate(wl, seed=3)
    d["idx"][:] = -1
    d["y"][:] = 0
    got, ref, _ = _case(wl, d=d)
    assert int(got["expert_offset"][-1]) == 0 and np.all(got["out"] == 0)


@pytest.mark.parametrize("fused", [False, True])
def test_empty_batch(fused):
    """T = 0 through ep_layout + ep_dispatch + ep_combine, and through
    ep_layout_dispatch (which takes the same guarded one-wave layout kernel
    and enqueues no dispatch): zero counts and offsets, clean status."""
    wl = WORKLOADS["tiny_4x1024"].with_(name="edge_T0", T=0)
    d = generate(wl, seed=1)
    print("case edge_T0 fused=%s" % fused, flush=True)
    got = run_gpu(wl, d, fused=fused)
    assert np.all(got["expert_count"] == 0) and np.all(got["expert_offset"] == 0)
    assert np.all(got["part_offset"] == 0) and int(got["status"][0]) == 0


def test_hot_expert_over_chunks():
    """Every entry of a large batch on one expert: the chunked layout's
    per-chunk bases carry a single expert's rows across every chunk."""
    wl = WORKLOADS["masked_16384x4096_bf16"].with_(name="edge_hot", T=2048, H=256, mask_frac=0.0)
    d = generate(wl, seed=9)
    d["idx"][:, 0] = 5
    _case(wl, d=d)


def test_deterministic_repeat():
    wl = WORKLOADS["bw_4096x7168_zipf"].with_(T=512)
    d = generate(wl)
    a = run_gpu(wl, d)
    b = run_gpu(wl, d)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_fp8_quotient_sweep():
    """Blocks whose amax sweeps the whole bf16 range (including scales below
    2^-90, which take the IEEE-division path, mixed with the shortcut path
    inside the same wave), with every other element a random bf16 of at most
    that magnitude: fp8 bytes and scales bit-exact against the oracle."""
    T, H, K, E, P = 2048, 2048, 1, 8, 1
    wl = WORKLOADS["tiny_4x1024"].with_(name="fp8_quotient_sweep", T=T, H=H, K=K, E=E, P=P)
    rng = np.random.default_rng(2024)
    nblk = T * H // 128
    amax_code = (1 + (np.arange(nblk, dtype=np.int64) * 997) % 0x7F7F).astype(np.uint16)
    codes = (rng.random((nblk, 128)) * (amax_code[:, None].astype(np.float64) + 1)).astype(np.uint32)
    codes = np.minimum(codes, amax_code[:, None]).astype(np.uint16)
    codes[:, 0] = amax_code
    signs = (rng.random((nblk, 128)) < 0.5).astype(np.uint16) << 15
    x = (codes | signs).reshape(T, H)
    d = dict(idx=(np.arange(T, dtype=np.int32) % E).reshape(T, 1), w=np.ones((T, 1), np.float32),
             x=x, y=np.zeros((T, H), np.uint16), N=T)
    _case(wl, d=d)


@pytest.mark.parametrize("fused", [False, True])
def test_fp8_non_finite_inputs(fused):
    """Non-finite hidden values (outside the parity workloads; the documented
    reading of the pages' silence): amax is a NaN-ignoring max starting from
    0, so a NaN element leaves its block's scale finite and encodes to NaN
    itself, and an all-NaN block gets scale 0 and zero bytes; an infinite
    element makes the scale infinite, the other elements of its block encode
    to signed zero and the infinite one (inf / inf) to NaN.  Layout, scales
    and bytes match the oracle bit for bit, except that the sign of a NaN
    byte is not compared: the host's and the device's default NaN differ in
    sign."""
    T, H, K, E, P = 64, 1024, 2, 8, 2
    wl = WORKLOADS["tiny_4x1024"].with_(name="fp8_non_finite", T=T, H=H, K=K, E=E, P=P)
    d = generate(wl, seed=31)
    x = d["x"].copy().reshape(T, H // 128, 128)
    rng = np.random.default_rng(31)
    NAN, NNAN, INF, NINF = 0x7FC0, 0xFFC0, 0x7F80, 0xFF80
    for t in range(T):
        j = rng.integers(0, 128, size=4)
        x[t, 0, j[0]] = NAN if t % 2 else NNAN       # one NaN among finite values
        x[t, 1, :] = NAN                             # all NaN
        x[t, 2, j[1]] = INF                          # one +inf
        x[t, 3, j[2]] = NINF                         # one -inf
        x[t, 4, j[0]] = NNAN                         # NaN and inf together
        x[t, 4, j[3]] = INF if j[3] != j[0] else x[t, 4, j[3]]
        x[t, 5, :] = 0                               # NaN among zeros: amax 0
        x[t, 5, j[1]] = NAN
        x[t, 6, j[2]] = INF                          # +inf and -inf
        x[t, 6, (j[2] + 1) % 128] = NINF
    d["x"] = x.reshape(T, H)
    got = run_gpu(wl, d, fused=fused)
    ref = run_oracle(wl, d)
    for k in ("expert_count", "expert_offset", "part_count", "part_offset", "row_of_pair",
              "src_pair"):
        np.testing.assert_array_equal(got[k], ref[k], err_msg=k)
    N = int(ref["expert_offset"][E])
    gx, rx = got["recv_x"][:N].astype(np.int32), ref["recv_x"][:N].astype(np.int32)
    nan_ref = (rx & 0x7F) == 0x7F
    assert np.array_equal(nan_ref, (gx & 0x7F) == 0x7F), "NaN bytes at different places"
    assert np.array_equal(gx[~nan_ref], rx[~nan_ref]), "finite bytes differ"
    assert nan_ref.any() and (rx[~nan_ref] & 0x7F == 0).any()
    gs, rs = got["recv_scales"][:N], ref["recv_scales"][:N]
    both_nan = np.isnan(gs) & np.isnan(rs)
    assert np.array_equal(gs.view(np.uint32)[~both_nan], rs.view(np.uint32)[~both_nan])
    assert np.isinf(rs).any() and (rs == 0).any()


def test_bound_step_matches_oracle():
    """BoundStep (arguments marshalled once) gives the same outputs as the
    oracle, call after call."""
    import torch
    import combine_ep_layout_05_amd as ep
    from tests.pathrun import collect, to_dev
    wl = WORKLOADS["ll_128x7168"]
    d = generate(wl, seed=wl.seed + 7)
    buf = ep.EpBuffers(wl.T, wl.H, wl.K, wl.E, wl.P, payload=wl.payload)
    idx, w = to_dev(d["idx"]), to_dev(d["w"])
    x = to_dev(d["x"].view(np.int16), torch.bfloat16)
    y = to_dev(d["y"].view(np.int16), torch.bfloat16)
    bs = ep.BoundStep(buf, idx, x, y, w)
    ref = run_oracle(wl, d)
    for _ in range(3):
        buf.out.zero_()
        bs.step()
        torch.cuda.synchronize()
        assert compare(wl, collect(buf), ref, check_poison=False) == 0


@pytest.mark.parametrize("fused", [False, True])
def test_masked_entries_never_use_row0(fused):
    """For a masked entry the combine reads row 0 of the expert outputs (an
    in-bounds stand-in) and must not add it: row 0 is +inf here, so a token
    that used it for a masked entry would come out infinite.  Only tokens
    that own row 0 through a valid entry may be infinite, exactly as in the
    oracle."""
    wl = WORKLOADS["tiny_4x1024"].with_(name="row0_inf", T=40, H=1024, E=64, P=8, K=8)
    d = generate(wl, seed=31)
    rng = np.random.default_rng(31)
    idx = d["idx"].copy()
    idx[rng.random(idx.shape) < 0.25] = -1
    d["idx"] = idx
    y = d["y"].copy()
    y[0, :] = 0x7F80                                    # bf16 +inf
    d["y"] = y
    got, ref, _ = _case(wl, d=d, fused=fused)
    owner = np.nonzero(ref["row_of_pair"] == 0)[0] // wl.K
    inf_tok = np.nonzero(np.isinf(bf16_to_f32(got["out"])).any(axis=1))[0]
    assert set(inf_tok.tolist()) <= set(owner.tolist())
