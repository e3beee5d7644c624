"""GPU test of ep_layout_dispatch_noalloc, the entry point that allocates
nothing: through the C ABI, on two calls in a row (the second with a smaller
batch, both large enough to need the layout workspace, i.e. the library's
scratch buffer), against ep_layout_dispatch with a caller-allocated workspace
on the same inputs.  The bar is the layout's and the dispatch's: every
output bit for bit.  A third call at a fused size (no workspace) checks the
path that does not touch the scratch buffer."""
import sys

import numpy as np
import pytest
import torch

from tests.pathrun import POISON_BYTE, POISON_F32_BITS, to_dev
from workloads import WORKLOADS, generate

pytestmark = pytest.mark.gpu

KEYS = ("expert_count", "expert_offset", "part_count", "part_offset", "row_of_pair", "src_pair",
        "status", "recv_x", "recv_scales")


def _buffers(ep, wl):
    buf = ep.EpBuffers(wl.T, wl.H, wl.K, wl.E, wl.P, payload=wl.payload)
    buf.recv_x.view(torch.uint8).fill_(POISON_BYTE)
    if buf.recv_scales is not None:
        buf.recv_scales.view(torch.int32).fill_(POISON_F32_BITS)
    for t in (buf.row_of_pair, buf.src_pair, buf.expert_count, buf.expert_offset):
        t.fill_(-7)
    return buf


def _outputs(buf):
    return {k: getattr(buf, k).view(torch.uint8).cpu().numpy() if k in ("recv_x",) else
            getattr(buf, k).cpu().numpy() for k in KEYS if getattr(buf, k) is not None}


def _pair(wl, seed, stream):
    import combine_ep_layout_05_amd as ep
    print("case %s T=%d H=%d K=%d E=%d P=%d %s workspace %d B" % (
        wl.name, wl.T, wl.H, wl.K, wl.E, wl.P, wl.payload,
        ep.ep_layout_workspace_bytes(wl.T, wl.K, wl.E)), flush=True)
    sys.stdout.flush()
    d = generate(wl, seed=seed)
    idx = to_dev(d["idx"])
    x = to_dev(d["x"].view(np.int16), torch.bfloat16)
    ref = _buffers(ep, wl)
    ref.layout_dispatch(idx, x, stream)
    got = _buffers(ep, wl)
    ep.ep_layout_dispatch_noalloc(idx, x, wl.E, wl.P, wl.payload, got.expert_count,
                                  got.expert_offset, got.part_count, got.part_offset,
                                  got.row_of_pair, got.src_pair, got.status, got.recv_x,
                                  got.recv_scales, stream)
    torch.cuda.synchronize()
    a, b = _outputs(got), _outputs(ref)
    for k in b:
        np.testing.assert_array_equal(a[k], b[k], err_msg="%s: %s" % (wl.name, k))
    return int(b["expert_offset"][wl.E])


def test_noalloc_matches_layout_dispatch_two_calls_then_smaller():
    import combine_ep_layout_05_amd as ep
    stream = torch.cuda.Stream()
    base = WORKLOADS["tiny_4x1024"]
    big = base.with_(name="noalloc_big", T=1024, H=1024, E=256, P=8)        # 8192 entries, 8 chunks
    small = base.with_(name="noalloc_small", T=600, H=640, E=96, P=4, mask_frac=0.1)   # 4800 entries
    fused = base.with_(name="noalloc_fused", T=64, H=7168, E=288, P=16)     # no workspace needed
    for wl in (big, small):
        assert ep.ep_layout_workspace_bytes(wl.T, wl.K, wl.E) > 0
    assert ep.ep_layout_workspace_bytes(fused.T, fused.K, fused.E) == 0
    assert _pair(big, 11, stream) > 0
    assert _pair(small, 12, stream) > 0
    assert _pair(fused, 13, stream) > 0


def test_noalloc_bf16_and_repeat():
    stream = torch.cuda.Stream()
    wl = WORKLOADS["tiny_4x1024"].with_(name="noalloc_bf16", T=700, H=512, E=128, P=8,
                                        payload="bf16")
    _pair(wl, 21, stream)
    _pair(wl.with_(name="noalloc_bf16_small", T=520), 22, stream)


def test_noalloc_rejects_batches_beyond_the_scratch_buffer():
    """E = 1024 and 2^20 + 2^17 entries need more than EP_NOALLOC_SCRATCH_BYTES:
    rejected with EP_ESCRATCH on the host before anything is enqueued (the
    argument checks pass with real, correctly sized buffers)."""
    import combine_ep_layout_05_amd as ep
    T, K, E, P, H = 73728, 16, 1024, 8, 128
    assert ep.ep_layout_workspace_bytes(T, K, E) > ep.EP_NOALLOC_SCRATCH_BYTES
    i32 = dict(dtype=torch.int32, device="cuda")
    idx = torch.zeros((T, K), **i32)
    x = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    outs = [torch.empty(E, **i32), torch.empty(E + 1, **i32), torch.empty(P, **i32),
            torch.empty(P + 1, **i32), torch.empty(T * K, **i32), torch.empty(T * K, **i32),
            torch.empty(1, **i32)]
    recv_x = torch.empty((T * K, H), dtype=torch.uint8, device="cuda")
    recv_s = torch.empty((T * K, H // 128), dtype=torch.float32, device="cuda")
    with pytest.raises(ep.EpError) as ei:
        ep.ep_layout_dispatch_noalloc(idx, x, E, P, "fp8", *outs, recv_x, recv_s)
    assert ei.value.code == ep.EP_ESCRATCH
    torch.cuda.synchronize()
