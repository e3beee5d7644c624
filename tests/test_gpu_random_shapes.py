"""GPU parity on seeded random shapes: T, H, E, P, K and payload drawn within
the API's limits (both layout regimes, both dispatch launches, partial
512-column steps), for the plain path (separate calls and the fused call) and
the per-destination path, each against the oracle."""
import numpy as np
import pytest

from tests.pathrun import (compare, compare_dedup, run_gpu, run_gpu_dedup, run_oracle,
                           run_oracle_dedup)
from workloads import WORKLOADS, generate

pytestmark = pytest.mark.gpu


def _shapes(n, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        K = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16]))
        P = int(rng.choice([1, 2, 3, 4, 8, 16]))
        L = int(rng.integers(1, 65))
        E = min(P * L, 1024 // P * P)
        E = max(E, P)
        if K > E:
            K = E
        payload = "bf16" if rng.random() < 0.3 else "fp8"
        H = int(rng.integers(1, 41)) * (8 if payload == "bf16" else 128)
        T = int(rng.choice([1, 2, 5, 17, 64, 129, 300, 700]))
        out.append(dict(name="rand%02d" % i, T=T, H=H, E=E, P=P, K=K, payload=payload,
                        mask_frac=float(rng.choice([0.0, 0.05]))))
    return out


SHAPES = _shapes(64)


@pytest.mark.parametrize("shape", SHAPES, ids=[s["name"] for s in SHAPES])
def test_random_shape_parity(shape):
    wl = WORKLOADS["tiny_4x1024"].with_(**shape)
    print("random shape", shape, flush=True)
    d = generate(wl, seed=500 + int(shape["name"][4:]))
    ref = run_oracle(wl, d)
    for fused in (False, True):
        got = run_gpu(wl, d, fused=fused)
        assert compare(wl, got, ref) == 0, (shape, fused)
    dref = run_oracle_dedup(wl, d)
    for fused in (False, True):
        got = run_gpu_dedup(wl, d, fused=fused)
        assert compare_dedup(wl, got, dref) == 0, (shape, fused)
