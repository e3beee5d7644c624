"""Buffers sized for T tokens serve batches of n <= T: each call works on the
first rows of the same buffers and gives, bit for bit, what buffers sized for
exactly n give (those are checked against the oracle elsewhere); batches of
different sizes follow one another, the last layout setting the size."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _inputs(T, H, E, P, K, payload, seed):
    from workloads import WORKLOADS, generate
    wl = WORKLOADS["tiny_4x1024"].with_(name="batch", T=T, H=H, E=E, P=P, K=K, payload=payload,
                                        mask_frac=0.05)
    d = generate(wl, seed=seed)
    dev = "cuda"
    return (torch.from_numpy(d["idx"]).to(dev),
            torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).to(dev),
            torch.from_numpy(d["y"].view(np.int16)).view(torch.bfloat16).to(dev),
            torch.from_numpy(d["w"]).to(dev))


def _plain(buf, idx, x, y, w, fused):
    if fused:
        buf.layout_dispatch(idx, x)
    else:
        buf.layout(idx)
        buf.dispatch(x)
    out = buf.combine(y, w)
    torch.cuda.synchronize()
    n, K = idx.shape
    N = int(buf.expert_offset[buf.E])
    r = {k: getattr(buf, k).clone() for k in ("expert_count", "expert_offset", "part_count",
                                                 "part_offset", "status")}
    r["row_of_pair"] = buf.row_of_pair[:n * K].clone()
    r["src_pair"] = buf.src_pair[:n * K].clone()
    r["rows"] = buf.recv_x[:N].clone()
    if buf.recv_scales is not None:
        r["scales"] = buf.recv_scales[:N].clone()
    r["out"] = out.clone()
    return r


@pytest.mark.parametrize("payload", ["fp8", "bf16"])
@pytest.mark.parametrize("fused", [True, False])
def test_plain_batches_below_capacity(payload, fused):
    import combine_ep_layout_05_amd as ep
    T, H, E, P, K = 300, 1024, 64, 8, 8
    big = ep.EpBuffers(T, H, K, E, P, payload=payload)
    for n, seed in ((300, 1), (37, 2), (5, 3), (129, 4), (300, 5)):
        print("plain batch n=%d of %d %s fused=%s" % (n, T, payload, fused), flush=True)
        idx, x, y, w = _inputs(n, H, E, P, K, payload, seed)
        got = _plain(big, idx, x, y, w, fused)
        ref = _plain(ep.EpBuffers(n, H, K, E, P, payload=payload), idx, x, y, w, fused)
        assert big.n == n
        for k in ref:
            assert torch.equal(got[k], ref[k]), (n, k)


def test_dedup_batches_below_capacity():
    import combine_ep_layout_05_amd as ep
    T, H, E, P, K = 200, 1024, 64, 8, 8
    big_p = ep.EpBuffers(T, H, K, E, P)
    big_d = ep.EpDedupBuffers(T, H, K, E, P)
    for n, seed in ((200, 11), (23, 12), (4, 13), (200, 14)):
        print("dedup batch n=%d of %d" % (n, T), flush=True)
        idx, x, y, w = _inputs(n, H, E, P, K, "fp8", seed)
        res = []
        for bp, bd in ((big_p, big_d), (ep.EpBuffers(n, H, K, E, P), ep.EpDedupBuffers(n, H, K, E, P))):
            bd.layout_dispatch(idx, x, bp)
            bd.combine_partial(y, bp.row_of_pair, w)
            out = bd.combine_reduce()
            torch.cuda.synchronize()
            M = int(bd.part_token_offset[P])
            res.append({"tp_row": bd.tp_row[:n * P].clone(), "kmask": bd.kmask[:n * P].clone(),
                        "rows": bd.recv_x[:M].clone(), "scales": bd.recv_scales[:M].clone(),
                        "row_of_pair": bp.row_of_pair[:n * K].clone(), "out": out.clone()})
        assert big_d.n == n and big_p.n == n
        for k in res[1]:
            assert torch.equal(res[0][k], res[1][k]), (n, k)


def test_batch_size_checks():
    import combine_ep_layout_05_amd as ep
    b = ep.EpBuffers(16, 1024, 8, 64, 8)
    idx, x, y, w = _inputs(8, 1024, 64, 8, 8, "fp8", 21)
    b.layout_dispatch(idx, x)
    with pytest.raises(ValueError):
        b.combine(y, w[:4])                       # not the layout's 8 tokens
    big_idx, _, _, _ = _inputs(17, 1024, 64, 8, 8, "fp8", 22)
    with pytest.raises(ValueError):
        b.layout(big_idx)                         # more tokens than the buffers hold
    torch.cuda.synchronize()
