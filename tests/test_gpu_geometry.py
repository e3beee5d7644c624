"""GPU: every launch geometry the tuner may pick gives the same bytes.

ep_dispatch_geom / ep_combine_geom over all (waves_per_block, max_blocks)
candidates, plus a single one-wave workgroup striding over every item,
compared bit for bit with the default launch (itself checked against the
oracle), and once directly with the oracle.
"""
import numpy as np
import pytest

from tests.pathrun import POISON_BYTE, compare, run_oracle, to_dev
from workloads import WORKLOADS, generate

pytestmark = pytest.mark.gpu

SHAPES = {
    "ll_128x7168": WORKLOADS["ll_128x7168"],
    "ragged_H640_T33": WORKLOADS["tiny_4x1024"].with_(name="geom_ragged", T=33, H=640),
    "bf16_T300_H512": WORKLOADS["tiny_4x1024"].with_(name="geom_bf16", T=300, H=512, payload="bf16"),
}


def _run(wl, d, geometry):
    import torch
    import combine_ep_layout_05_amd as ep
    buf = ep.EpBuffers(wl.T, wl.H, wl.K, wl.E, wl.P, payload=wl.payload,
                       geometry={"dispatch": geometry, "combine": geometry})
    buf.recv_x.view(torch.uint8).fill_(POISON_BYTE)
    if buf.recv_scales is not None:
        buf.recv_scales.fill_(0.0)
    buf.out.view(torch.int16).fill_(0x5A5A)
    idx = to_dev(d["idx"])
    x = to_dev(d["x"].view(np.int16), torch.bfloat16)
    y = to_dev(d["y"].view(np.int16), torch.bfloat16)
    w = to_dev(d["w"])
    buf.layout(idx)
    buf.dispatch(x)
    buf.combine(y, w)
    torch.cuda.synchronize()
    from tests.pathrun import collect
    return collect(buf)


@pytest.mark.parametrize("shape", list(SHAPES))
def test_all_geometries_bit_identical(shape):
    import combine_ep_layout_05_amd.tuning as tu
    wl = SHAPES[shape]
    d = generate(wl, seed=wl.seed + 31)
    print("geometry parity %s T=%d H=%d %s" % (wl.name, wl.T, wl.H, wl.payload), flush=True)
    base = _run(wl, d, None)
    assert compare(wl, base, run_oracle(wl, d), check_poison=True) == 0
    for geom in tu.candidates() + [(1, 1), (8, 1), (2, 3)]:
        got = _run(wl, d, geom)
        for k in base:
            assert np.array_equal(got[k], base[k]), (shape, geom, k)


def test_geometry_rejected_on_host():
    import torch
    import combine_ep_layout_05_amd as ep
    buf = ep.EpBuffers(4, 1024, 8, 32, 8)
    x = torch.zeros(4, 1024, dtype=torch.bfloat16, device="cuda")
    for bad in [(3, 0), (16, 0), (0, 0), (4, -1)]:
        with pytest.raises(ep.EpError):
            ep.ep_dispatch(x, 8, buf.row_of_pair, "fp8", buf.recv_x, buf.recv_scales, None, bad)
