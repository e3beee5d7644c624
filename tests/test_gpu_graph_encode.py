"""GPU: HIP-graph replay against eager execution, and the device e4m3fn
encoder against the oracle's encoder over whole ranges of fp32 inputs."""
import sys

import numpy as np
import pytest
import torch

import oracle
from tests.pathrun import collect, compare, run_oracle, to_dev
from workloads import WORKLOADS, generate

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("name", ["sweep_4x6144", "ll_128x7168", "bw_4096x7168_zipf"])
def test_graph_replay_matches_eager(name, fused):
    """A captured layout -> dispatch -> combine step replays bit-exactly to the
    eager result, replay after replay, with unrelated eager work and
    synchronisations in between (the check MoRI PR #614 runs for its
    dispatch/combine under HIP graphs)."""
    import combine_ep_layout_05_amd as ep
    wl = WORKLOADS[name]
    if wl.T > 1024:
        wl = wl.with_(T=1024)
    print("graph case", wl.name, wl.T, flush=True)
    d = generate(wl)
    idx, w = to_dev(d["idx"]), to_dev(d["w"])
    x = to_dev(d["x"].view(np.int16), torch.bfloat16)
    y = to_dev(d["y"].view(np.int16), torch.bfloat16)

    eager = ep.EpBuffers(wl.T, wl.H, wl.K, wl.E, wl.P, payload=wl.payload)
    eager.layout(idx)
    eager.dispatch(x)
    eager.combine(y, w)
    torch.cuda.synchronize()
    ref = collect(eager)
    compare(wl, ref, run_oracle(wl, d), check_poison=False)

    buf = ep.EpBuffers(wl.T, wl.H, wl.K, wl.E, wl.P, payload=wl.payload)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ep.ep_graph_begin(s)
        if fused:
            buf.layout_dispatch(idx, x, s)
        else:
            buf.layout(idx, s)
            buf.dispatch(x, s)
        buf.combine(y, w, s)
        g = ep.ep_graph_end(s)
    replay = g.bind(s)                   # the bound form: odd replays
    for rep in range(4):
        buf.recv_x.view(torch.uint8).fill_(0)
        buf.out.zero_()
        buf.row_of_pair.fill_(-5)
        junk = torch.randn(1 << 20, device="cuda").sum()     # unrelated eager work
        torch.cuda.synchronize()
        if rep % 2 == 0:
            g.launch(s)
        else:
            replay()
        s.synchronize()
        got = collect(buf)
        for k in ref:
            assert np.array_equal(got[k], ref[k]), "replay %d: %s" % (rep, k)
        del junk
    g.destroy()


def test_graph_replay_of_a_batch_below_capacity():
    """Buffers for 256 tokens, a captured step of a 40-token batch (int64 ids:
    the narrowing launch is captured too): every replay equals the eager
    40-token step, with unrelated eager work in between, and leaves the rows
    past the batch alone."""
    import combine_ep_layout_05_amd as ep
    wl = WORKLOADS["ll_128x7168"].with_(T=40)
    d = generate(wl, seed=77)
    idx64 = torch.from_numpy(d["idx"].astype(np.int64)).cuda()
    w = to_dev(d["w"])
    x = to_dev(d["x"].view(np.int16), torch.bfloat16)
    y = to_dev(d["y"].view(np.int16), torch.bfloat16)
    print("graph case below capacity: 40 of 256 tokens", flush=True)
    eager = ep.EpBuffers(wl.T, wl.H, wl.K, wl.E, wl.P, payload=wl.payload)
    eager.layout_dispatch(idx64, x)
    eager.combine(y, w)
    torch.cuda.synchronize()
    ref = collect(eager)
    compare(wl, ref, run_oracle(wl, d), check_poison=False)

    buf = ep.EpBuffers(256, wl.H, wl.K, wl.E, wl.P, payload=wl.payload)
    m = wl.T * wl.K
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ep.ep_graph_begin(s)
        buf.layout_dispatch(idx64, x, s)
        buf.combine(y, w, s)
        g = ep.ep_graph_end(s)
    for rep in range(3):
        buf.recv_x.view(torch.uint8).fill_(0)
        buf.out.zero_()
        buf.row_of_pair.fill_(-5)
        junk = torch.randn(1 << 20, device="cuda").sum()     # unrelated eager work
        torch.cuda.synchronize()
        g.launch(s)
        s.synchronize()
        got = collect(buf, wl.T)
        for k in ref:
            assert np.array_equal(got[k], ref[k]), "replay %d: %s" % (rep, k)
        assert bool((buf.row_of_pair[m:] == -5).all()), "replay %d: rows past the batch" % rep
        assert bool((buf.out[wl.T:].view(torch.int16) == 0).all())
        del junk
    g.destroy()


@pytest.mark.parametrize("name", ["ll_128x7168", "bw_4096x7168_zipf"])
def test_dedup_graph_replay_matches_eager(name):
    """The per-destination step (ep_dedup_layout_dispatch, ep_combine_partial,
    ep_combine_reduce), captured once, replays bit-exactly to the eager result
    with unrelated eager work in between; the small batch runs the one-launch
    path, the 1024-token batch the three-kernel path."""
    import combine_ep_layout_05_amd as ep
    wl = WORKLOADS[name]
    if wl.T > 1024:
        wl = wl.with_(T=1024)
    print("dedup graph case", wl.name, wl.T, flush=True)
    d = generate(wl)
    idx, w = to_dev(d["idx"]), to_dev(d["w"])
    x = to_dev(d["x"].view(np.int16), torch.bfloat16)
    y = to_dev(d["y"].view(np.int16), torch.bfloat16)

    def run(buf, db, s=None):
        db.layout_dispatch(idx, x, buf, s)
        db.combine_partial(y, buf.row_of_pair, w, s)
        db.combine_reduce(s)

    def grab(buf, db):
        torch.cuda.synchronize()
        r = {k: getattr(db, k).cpu().numpy().copy() for k in
             ("tp_row", "part_tokens", "part_token_offset", "tp_src", "kmask", "status")}
        M = int(r["part_token_offset"][wl.P])
        r["recv_x"] = db.recv_x.view(torch.uint8).cpu().numpy()[:M].copy()
        r["partial"] = db.partial.view(torch.int16).cpu().numpy()[:M].copy()
        r["out"] = db.out.view(torch.int16).cpu().numpy().copy()
        r["row_of_pair"] = buf.row_of_pair.cpu().numpy().copy()
        return r

    b0 = ep.EpBuffers(wl.T, wl.H, wl.K, wl.E, wl.P, payload=wl.payload)
    d0 = ep.EpDedupBuffers(wl.T, wl.H, wl.K, wl.E, wl.P, payload=wl.payload)
    run(b0, d0)
    ref = grab(b0, d0)

    b1 = ep.EpBuffers(wl.T, wl.H, wl.K, wl.E, wl.P, payload=wl.payload)
    d1 = ep.EpDedupBuffers(wl.T, wl.H, wl.K, wl.E, wl.P, payload=wl.payload)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ep.ep_graph_begin(s)
        run(b1, d1, s)
        g = ep.ep_graph_end(s)
    for rep in range(4):
        d1.recv_x.view(torch.uint8).fill_(0)
        d1.partial.zero_()
        d1.out.zero_()
        d1.tp_row.fill_(-5)
        b1.row_of_pair.fill_(-5)
        junk = torch.randn(1 << 20, device="cuda").sum()     # unrelated eager work
        torch.cuda.synchronize()
        g.launch(s)
        s.synchronize()
        got = grab(b1, d1)
        for k in ref:
            assert np.array_equal(got[k], ref[k]), "replay %d: %s" % (rep, k)
        del junk
    g.destroy()


def test_device_encoder_against_oracle_ranges():
    """All fp32 bit patterns with magnitude in [2^-12, 512) (both signs), plus
    the special values: the device encoder equals the oracle's."""
    import combine_ep_layout_05_amd as ep
    lo = int(np.float32(2.0 ** -12).view(np.uint32))
    hi = int(np.float32(512.0).view(np.uint32))
    step = 1 << 24
    for b0 in range(lo, hi, step):
        bits = np.arange(b0, min(b0 + step, hi), dtype=np.uint32)
        for sign in (0, 0x80000000):
            v = (bits | np.uint32(sign)).view(np.float32)
            dv = torch.from_numpy(v).cuda()
            out = torch.empty(v.size, dtype=torch.uint8, device="cuda")
            ep.ep_e4m3fn_encode(dv, out)
            got = out.cpu().numpy()
            ref = oracle.e4m3fn_encode(v)
            bad = np.nonzero(got != ref)[0]
            assert bad.size == 0, (hex(int(v.view(np.uint32)[bad[0]])), hex(got[bad[0]]), hex(ref[bad[0]]))
        print("encoder range up to %s ok" % hex(b0 + step), flush=True)
        sys.stdout.flush()
    special = np.array([0.0, -0.0, 448.0, -448.0, 449.0, 464.0, 465.0, 1e30, -1e30, np.inf, -np.inf,
                        1e-30, -1e-30, 2.0 ** -10, -(2.0 ** -10), 3 * 2.0 ** -10], np.float32)
    dv = torch.from_numpy(special).cuda()
    out = torch.empty(special.size, dtype=torch.uint8, device="cuda")
    ep.ep_e4m3fn_encode(dv, out)
    np.testing.assert_array_equal(out.cpu().numpy(), oracle.e4m3fn_encode(special))


def test_device_encoder_nan():
    """NaN encodes to 0x7F with the sign bit kept (documented behaviour; NaN
    inputs are outside the parity workloads)."""
    import combine_ep_layout_05_amd as ep
    nan_bits = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFA5A5A5], np.uint32)
    v = nan_bits.view(np.float32)
    out = torch.empty(4, dtype=torch.uint8, device="cuda")
    ep.ep_e4m3fn_encode(torch.from_numpy(v).cuda(), out)
    got = out.cpu().numpy()
    print("device NaN codes:", [hex(c) for c in got], flush=True)
    np.testing.assert_array_equal(got & 0x7F, np.full(4, 0x7F, np.uint8))
