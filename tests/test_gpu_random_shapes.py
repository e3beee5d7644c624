"""GPU parity on seeded random shapes: T, H, E, P, K, payload and masking drawn
within the API's limits (every layout regime, both dispatch launches, partial
512-column steps), for the plain path (separate calls, the fused call, and the
fused call with a random geometry its plan accepts) and the per-destination
path (the same three), each against the oracle; two of each three through
buffers for more tokens than the batch (up to 300 more), whose rows past the
batch must stay untouched.

64 shapes by default; EP_RANDOM_SHAPES and EP_RANDOM_SEED draw more (or other)
shapes, e.g. EP_RANDOM_SHAPES=3000 for a long sweep."""
import os

import numpy as np
import pytest

from tests.pathrun import (compare, compare_dedup, run_gpu, run_gpu_dedup, run_oracle,
                           run_oracle_dedup)
from workloads import WORKLOADS, generate

pytestmark = pytest.mark.gpu

COUNT = int(os.environ.get("EP_RANDOM_SHAPES") or "64")
SEED = int(os.environ.get("EP_RANDOM_SEED") or "2024")


def _shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        K = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 12, 16]))
        P = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
        L = int(rng.integers(1, 65))
        E = max(min(P * L, 1024 // P * P), P)
        K = min(K, E)
        payload = "bf16" if rng.random() < 0.3 else "fp8"
        H = int(rng.integers(1, 57)) * (8 if payload == "bf16" else 128)
        T = int(rng.choice([1, 2, 3, 4, 7, 16, 33, 64, 100, 128, 129, 200, 256, 300, 511, 700]))
        out.append(dict(name="rand%04d" % i, T=T, H=H, E=E, P=P, K=K, payload=payload,
                        mask_frac=float(rng.choice([0.0, 0.05, 0.3])),
                        pick=int(rng.integers(1 << 30)), dpick=int(rng.integers(1 << 30)),
                        extra=int(rng.choice([0, 0, 1, 7, 64, 300]))))
    return out


SHAPES = _shapes(COUNT, SEED)


@pytest.mark.parametrize("shape", SHAPES, ids=[s["name"] for s in SHAPES])
def test_random_shape_parity(shape):
    from combine_ep_layout_05_amd import tuning
    sh = {k: v for k, v in shape.items() if k not in ("pick", "dpick", "extra")}
    cap = shape["T"] + shape["extra"]             # buffers for more tokens than the batch
    wl = WORKLOADS["tiny_4x1024"].with_(**sh)
    dims = dict(T=wl.T, H=wl.H, K=wl.K, E=wl.E, P=wl.P, payload=wl.payload)
    cands = tuning.candidates("layout_dispatch", dims)
    geom = cands[shape["pick"] % len(cands)]
    dcands = tuning.candidates("dedup_layout_dispatch", dims)
    dgeom = dcands[shape["dpick"] % len(dcands)]
    print("random shape", sh, "capacity", cap, "geometry", geom, "dedup geometry", dgeom,
          flush=True)
    d = generate(wl, seed=500 + int(shape["name"][4:]) + SEED)
    ref = run_oracle(wl, d)
    for fused, g, c in ((False, None, cap), (True, None, None), (True, {"layout_dispatch": geom}, cap)):
        got = run_gpu(wl, d, fused=fused, geometry=g, capacity=c)
        assert compare(wl, got, ref) == 0, (shape, fused, g, c)
    dref = run_oracle_dedup(wl, d)
    for fused, g, c in ((False, None, cap), (True, None, None), (True, dgeom, cap)):
        got = run_gpu_dedup(wl, d, fused=fused, geometry=g, capacity=c)
        assert compare_dedup(wl, got, dref) == 0, (shape, fused, g, c)
