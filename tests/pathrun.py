"""Runs the HIP path and the oracle on the same seeded inputs, for the tests.

GPU side: the C-ABI library through its thin Python binding.  Oracle side:
oracle/ (CPU).  The two share nothing but the inputs from workloads/.
"""
import numpy as np
import torch

import oracle

POISON_BYTE = 0xA5
POISON_F32_BITS = 0x7FA5A5A5          # a NaN pattern no kernel writes


def gpu_lib():
    import combine_ep_layout_05_amd as ep
    return ep


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def run_gpu(wl, d, stream=None, poison=True, fused=False, geometry=None, capacity=None):
    """Layout + dispatch + combine on the GPU; returns numpy copies of every output.
    fused=True runs ep_layout_dispatch instead of ep_layout then ep_dispatch;
    geometry is EpBuffers' launch geometry (None: the library default);
    capacity: buffers for that many tokens (>= wl.T) holding the batch in
    their first rows, the rest checked to stay untouched."""
    ep = gpu_lib()
    cap = wl.T if capacity is None else capacity
    buf = ep.EpBuffers(cap, wl.H, wl.K, wl.E, wl.P, payload=wl.payload, geometry=geometry)
    if poison:
        buf.recv_x.view(torch.uint8).fill_(POISON_BYTE)
        if buf.recv_scales is not None:
            buf.recv_scales.view(torch.int32).fill_(POISON_F32_BITS)
        buf.row_of_pair.fill_(-7)
        buf.src_pair.fill_(-7)
        buf.out.view(torch.int16).fill_(0x5A5A)
    idx = to_dev(d["idx"])
    x = to_dev(d["x"].view(np.int16), torch.bfloat16)
    y = to_dev(d["y"].view(np.int16), torch.bfloat16)
    w = to_dev(d["w"])
    if fused:
        buf.layout_dispatch(idx, x, stream)
    else:
        buf.layout(idx, stream)
        buf.dispatch(x, stream)
    buf.combine(y, w, stream)
    torch.cuda.synchronize()
    if poison and cap > wl.T:
        m = wl.T * wl.K
        assert bool((buf.recv_x[m:].view(torch.uint8) == POISON_BYTE).all()), "recv_x past the batch"
        assert bool((buf.row_of_pair[m:] == -7).all()) and bool((buf.src_pair[m:] == -7).all())
        assert bool((buf.out[wl.T:].view(torch.int16) == 0x5A5A).all()), "out past the batch"
    return collect(buf, wl.T)


def collect(buf, T=None):
    T = buf.T if T is None else T
    m = T * buf.K
    res = {k: getattr(buf, k).cpu().numpy() for k in
           ("expert_count", "expert_offset", "part_count", "part_offset")}
    res["row_of_pair"] = buf.row_of_pair[:m].cpu().numpy()
    res["src_pair"] = buf.src_pair[:m].cpu().numpy()
    res["status"] = buf.status.cpu().numpy().view(np.uint32)
    res["recv_x"] = buf.recv_x[:m].view(torch.uint8).cpu().numpy() if buf.payload == "fp8" else \
        buf.recv_x[:m].view(torch.int16).cpu().numpy().view(np.uint16)
    if buf.recv_scales is not None:
        res["recv_scales"] = buf.recv_scales[:m].cpu().numpy()
    res["out"] = buf.out[:T].view(torch.int16).cpu().numpy().view(np.uint16)
    return res


def run_oracle(wl, d):
    lo = oracle.layout(d["idx"], wl.E, wl.P)
    res = dict(lo)
    if wl.payload == "fp8":
        rx, rs = oracle.dispatch_fp8(d["x"], lo["row_of_pair"], wl.K)
        res["recv_x"], res["recv_scales"] = rx, rs
    else:
        res["recv_x"] = oracle.dispatch_bf16(d["x"], lo["row_of_pair"], wl.K)
    res["out"] = oracle.combine(d["y"], lo["row_of_pair"], d["w"], wl.T, wl.H, wl.K)
    return res


def compare(wl, got, ref, check_poison=True):
    """Bit-exact for layout, fp8 bytes, scales, bf16 rows; combine within 1 bf16 ulp.
    Returns the number of combine outputs that differ at all (expected 0)."""
    from tests.helpers import bf16_ulp_distance
    for k in ("expert_count", "expert_offset", "part_count", "part_offset", "row_of_pair",
              "src_pair"):
        np.testing.assert_array_equal(got[k], ref[k], err_msg="%s: %s" % (wl.name, k))
    assert int(got["status"][0]) == int(ref["status"][0]), (wl.name, "status")
    N = int(ref["expert_offset"][wl.E])
    gx, rx = got["recv_x"], ref["recv_x"]
    bad = np.nonzero((gx[:N] != rx[:N]).any(axis=1))[0]
    assert bad.size == 0, "%s: recv_x rows differ, first row %d" % (wl.name, bad[0])
    if wl.payload == "fp8":
        gs = got["recv_scales"][:N].view(np.uint32)
        rs = ref["recv_scales"][:N].view(np.uint32)
        np.testing.assert_array_equal(gs, rs, err_msg="%s: recv_scales" % wl.name)
    if check_poison:
        tail = gx[N:].view(np.uint8)
        assert np.all(tail == POISON_BYTE), "%s: rows >= N were written" % wl.name
        if wl.payload == "fp8":
            assert np.all(got["recv_scales"][N:].view(np.uint32) == POISON_F32_BITS)
    dist = bf16_ulp_distance(got["out"], ref["out"])
    assert dist.max(initial=0) <= 1, "%s: combine off by %d ulp" % (wl.name, dist.max())
    return int(np.count_nonzero(dist))


DEDUP_KEYS = ("tp_row", "part_tokens", "part_token_offset", "tp_src", "kmask")


PLAIN_LAYOUT_KEYS = ("expert_count", "expert_offset", "part_count", "part_offset", "row_of_pair",
                     "src_pair")


def run_gpu_dedup(wl, d, stream=None, fused=False, geometry=None, capacity=None):
    """Per-destination path on the GPU: ep_layout (expert rows for the expert
    outputs), ep_dedup_layout, ep_dispatch with K = P over tp_row,
    ep_combine_partial and ep_combine_reduce; fused=True runs
    ep_dedup_layout_dispatch in place of the first three (with `geometry`,
    ep_dedup_layout_dispatch_geom).  Buffers start poisoned; capacity as in
    run_gpu."""
    ep = gpu_lib()
    cap = wl.T if capacity is None else capacity
    buf = ep.EpBuffers(cap, wl.H, wl.K, wl.E, wl.P, payload=wl.payload)
    db = ep.EpDedupBuffers(cap, wl.H, wl.K, wl.E, wl.P, payload=wl.payload)
    db.recv_x.view(torch.uint8).fill_(POISON_BYTE)
    if db.recv_scales is not None:
        db.recv_scales.view(torch.int32).fill_(POISON_F32_BITS)
    for t in (db.tp_row, db.tp_src, db.kmask, buf.row_of_pair, buf.src_pair):
        t.fill_(-7)
    db.partial.view(torch.int16).fill_(0x5A5A)
    db.out.view(torch.int16).fill_(0x5A5A)
    idx = to_dev(d["idx"])
    x = to_dev(d["x"].view(np.int16), torch.bfloat16)
    y = to_dev(d["y"].view(np.int16), torch.bfloat16)
    w = to_dev(d["w"])
    if fused:
        db.layout_dispatch(idx, x, buf, stream, geometry)
    else:
        buf.layout(idx, stream)
        db.layout(idx, stream)
        db.dispatch(x, stream)
    db.combine_partial(y, buf.row_of_pair, w, stream)
    db.combine_reduce(stream)
    torch.cuda.synchronize()
    T, mp, mk = wl.T, wl.T * wl.P, wl.T * wl.K
    if cap > T:
        assert bool((db.recv_x[mp:].view(torch.uint8) == POISON_BYTE).all()), "rows past the batch"
        for t in (db.tp_row[mp:], db.tp_src[mp:], db.kmask[mp:], buf.row_of_pair[mk:],
                  buf.src_pair[mk:]):
            assert bool((t == -7).all()), "maps past the batch"
        assert bool((db.partial[mp:].view(torch.int16) == 0x5A5A).all()), "partial past the batch"
        assert bool((db.out[T:].view(torch.int16) == 0x5A5A).all()), "out past the batch"
    res = {}
    for k in DEDUP_KEYS:
        t = getattr(db, k)
        res[k] = (t[:mp] if k in ("tp_row", "tp_src", "kmask") else t).cpu().numpy()
    res["kmask"] = res["kmask"].view(np.uint32)
    res["status"] = db.status.cpu().numpy().view(np.uint32)
    for k in PLAIN_LAYOUT_KEYS:
        t = getattr(buf, k)
        res[k] = (t[:mk] if k in ("row_of_pair", "src_pair") else t).cpu().numpy()
    res["recv_x"] = db.recv_x[:mp].view(torch.uint8).cpu().numpy() if wl.payload == "fp8" else \
        db.recv_x[:mp].view(torch.int16).cpu().numpy().view(np.uint16)
    if db.recv_scales is not None:
        res["recv_scales"] = db.recv_scales[:mp].cpu().numpy()
    res["partial"] = db.partial[:mp].view(torch.int16).cpu().numpy().view(np.uint16)
    res["out"] = db.out[:T].view(torch.int16).cpu().numpy().view(np.uint16)
    return res


def run_oracle_dedup(wl, d):
    lo = oracle.layout(d["idx"], wl.E, wl.P)
    dl = oracle.dedup_layout(d["idx"], wl.E, wl.P)
    res = dict(dl)
    for k in PLAIN_LAYOUT_KEYS:
        res[k] = lo[k]
    if wl.payload == "fp8":
        res["recv_x"], res["recv_scales"] = oracle.dispatch_fp8(d["x"], dl["tp_row"], wl.P)
    else:
        res["recv_x"] = oracle.dispatch_bf16(d["x"], dl["tp_row"], wl.P)
    res["partial"] = oracle.combine_partial(d["y"], lo["row_of_pair"], d["w"], dl["tp_row"],
                                            dl["kmask"], wl.T, wl.H, wl.K, wl.P)
    res["out"] = oracle.combine_reduce(res["partial"], dl["tp_row"], wl.T, wl.H, wl.P)
    return res


def compare_dedup(wl, got, ref):
    """Bit-exact layout, dispatch rows and scales; partial and output within
    1 bf16 ulp; rows past M untouched.  Returns the number of differing
    partial + output values (expected 0: same fmaf / add order)."""
    from tests.helpers import bf16_ulp_distance
    for k in DEDUP_KEYS + PLAIN_LAYOUT_KEYS:
        np.testing.assert_array_equal(got[k], ref[k], err_msg="%s: %s" % (wl.name, k))
    assert int(got["status"][0]) == int(ref["status"][0]), (wl.name, "status")
    M = int(ref["part_token_offset"][wl.P])
    gx, rx = got["recv_x"], ref["recv_x"]
    bad = np.nonzero((gx[:M] != rx[:M]).any(axis=1))[0]
    assert bad.size == 0, "%s: dedup recv_x rows differ, first row %d" % (wl.name, bad[0])
    assert np.all(gx[M:].view(np.uint8) == POISON_BYTE), "%s: rows >= M were written" % wl.name
    if wl.payload == "fp8":
        np.testing.assert_array_equal(got["recv_scales"][:M].view(np.uint32),
                                      ref["recv_scales"][:M].view(np.uint32))
        assert np.all(got["recv_scales"][M:].view(np.uint32) == POISON_F32_BITS)
    dp = bf16_ulp_distance(got["partial"][:M], ref["partial"][:M])
    assert dp.max(initial=0) <= 1, "%s: partial off by %d ulp" % (wl.name, dp.max())
    assert np.all(got["partial"][M:] == 0x5A5A), "%s: partial rows >= M were written" % wl.name
    do = bf16_ulp_distance(got["out"], ref["out"])
    assert do.max(initial=0) <= 1, "%s: output off by %d ulp" % (wl.name, do.max())
    return int(np.count_nonzero(dp)) + int(np.count_nonzero(do))
