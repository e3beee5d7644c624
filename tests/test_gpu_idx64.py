"""int64 expert ids: ep_topk_idx_narrow against its definition, and the
buffers' layout calls taking int64 ids give the outputs of the same int32
ids, bit for bit (a negative id drops the entry; one above INT32_MAX is a bad
id the status reports)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_topk_idx_narrow_values():
    import combine_ep_layout_05_amd as ep
    vals = np.array([0, 1, 287, 1023, 2**31 - 1, 2**31, 2**40, 2**63 - 1, -1, -2, -(2**31),
                     -(2**31) - 1, -(2**63)], dtype=np.int64)
    rng = np.random.default_rng(7)
    vals = np.concatenate([vals, rng.integers(-(2**62), 2**62, size=70000, dtype=np.int64),
                           rng.integers(-3, 300, size=5000, dtype=np.int64)])
    print("narrow n=%d" % vals.size, flush=True)
    src = torch.from_numpy(vals).cuda()
    out = torch.full((vals.size,), 12345, dtype=torch.int32, device="cuda")
    ep.ep_topk_idx_narrow(src, out)
    torch.cuda.synchronize()
    want = np.where(vals < 0, -1, np.minimum(vals, 2**31 - 1)).astype(np.int32)
    np.testing.assert_array_equal(out.cpu().numpy(), want)


@pytest.mark.parametrize("T,H,E,P,payload", [(128, 7168, 288, 16, "fp8"), (4, 6144, 256, 16, "fp8"),
                                             (600, 1024, 64, 8, "bf16")])
def test_buffers_take_int64_ids(T, H, E, P, payload):
    import combine_ep_layout_05_amd as ep
    from workloads import WORKLOADS, generate
    K = 8
    wl = WORKLOADS["tiny_4x1024"].with_(name="idx64", T=T, H=H, E=E, P=P, K=K, payload=payload,
                                        mask_frac=0.05)
    print("int64 ids T=%d H=%d E=%d P=%d %s" % (T, H, E, P, payload), flush=True)
    d = generate(wl, seed=31)
    idx = d["idx"].astype(np.int64)
    idx[0, 0] = 2**33                      # above INT32_MAX: a bad id
    idx[1, 1] = -(2**40)                   # a dropped entry
    idx32 = np.where(idx < 0, -1, np.minimum(idx, 2**31 - 1)).astype(np.int32)
    x = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).cuda()
    res = []
    for ids in (torch.from_numpy(idx).cuda(), torch.from_numpy(idx32).cuda()):
        b = ep.EpBuffers(T, H, K, E, P, payload=payload)
        b.layout_dispatch(ids, x)
        torch.cuda.synchronize()
        res.append({k: getattr(b, k).cpu().clone() for k in
                    ("expert_count", "expert_offset", "row_of_pair", "src_pair", "status")})
        N = int(res[-1]["expert_offset"][E])
        res[-1]["rows"] = b.recv_x[:N].cpu().clone()
    for k in res[0]:
        assert torch.equal(res[0][k], res[1][k]), k
    assert int(res[0]["status"][0]) & 1                          # the bad id is reported
    assert int(res[0]["row_of_pair"][1 * K + 1]) == -1             # the dropped entry
