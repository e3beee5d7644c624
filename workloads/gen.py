"""Workload table and seeded input generators.

Shapes follow the low-latency EP test shapes the sources quote: 128 tokens x
hidden 7168, top-8 of 288 experts (MoRI PR #614, test_low_latency.py argument
paragraph: defaults 128 / 7168 / 8 / 288); the 4/8/16-token, hidden-6144
serving regime (same PR, tuned-rules and view-cache paragraphs); an unbalanced
run where one destination takes 1.5x the mean load (DeepEP PR #693,
Validation: "rank unbalanced ratio 1.5"); and a large bf16 run with dropped
(-1) entries (negative sentinels: MoRI PR #614, routing-scan paragraph).

Random numbers: numpy's PCG64, one independent stream per tensor derived with
SeedSequence([seed, stream]), so a tensor's values do not depend on the sizes
of the others.  Normal values are drawn in fp32 and rounded to bf16 by torch's
round-to-nearest-even conversion.  Nothing here computes any part of the
dispatch/combine method.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np
import torch

# stream ids, one per generated tensor
_S_ROUTE, _S_MASK, _S_LOGIT, _S_X, _S_OUTLIER, _S_Y, _S_PERM = range(7)


@dataclass(frozen=True)
class Workload:
    name: str
    T: int                 # tokens
    H: int                 # hidden size
    E: int                 # experts
    P: int                 # destination partitions (stand-ins for EP ranks)
    K: int                 # top-k
    payload: str           # "fp8" (e4m3fn + per-128 fp32 scales) or "bf16" (passthrough)
    seed: int
    routing: str = "uniform"   # "uniform" distinct ids, or "zipf"
    zipf_s: float = 0.0
    part0_ratio: float = 0.0   # zipf: partition 0 load / mean partition load
    mask_frac: float = 0.0     # fraction of top-k entries set to -1 (exact count)
    outlier_frac: float = 0.0  # fraction of token rows scaled by outlier_scale
    outlier_scale: float = 1.0
    graph: bool = False        # timed as a captured graph (small-token regime)

    @property
    def L(self) -> int:
        return self.E // self.P

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _wl(*a, **k):
    w = Workload(*a, **k)
    return w.name, w


WORKLOADS = dict([
    _wl("tiny_4x1024", 4, 1024, 32, 8, 8, "fp8", seed=1),
    _wl("ll_128x7168", 128, 7168, 288, 16, 8, "fp8", seed=2,
        outlier_frac=0.01, outlier_scale=50.0),
    _wl("sweep_4x6144", 4, 6144, 256, 16, 8, "fp8", seed=3004, graph=True),
    _wl("sweep_8x6144", 8, 6144, 256, 16, 8, "fp8", seed=3008, graph=True),
    _wl("sweep_16x6144", 16, 6144, 256, 16, 8, "fp8", seed=3016, graph=True),
    _wl("bw_4096x7168_zipf", 4096, 7168, 256, 8, 8, "fp8", seed=4,
        routing="zipf", zipf_s=1.1, part0_ratio=1.5),
    _wl("masked_16384x4096_bf16", 16384, 4096, 128, 8, 8, "bf16", seed=5,
        mask_frac=0.10),
])


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, stream]))


def to_bf16_bits(a32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16) via torch's round-to-nearest-even cast."""
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _normal_bf16(rng: np.random.Generator, rows: int, cols: int, out=None) -> np.ndarray:
    """N(0,1) bf16 bits, generated in row chunks to bound host memory."""
    if out is None:
        out = np.empty((rows, cols), np.uint16)
    chunk = max(1, (1 << 23) // max(cols, 1))
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        out[r0:r1] = to_bf16_bits(rng.standard_normal((r1 - r0, cols), dtype=np.float32))
    return out


def uniform_distinct_routing(rng, T, E, K):
    """K distinct experts per token, uniformly at random (random-key shuffle)."""
    if T == 0:
        return np.zeros((0, K), np.int32)
    u = rng.random((T, E))
    return np.argsort(u, axis=1, kind="stable")[:, :K].astype(np.int32)


def zipf_routing(rng, perm_rng, T, E, P, K, s, part0_ratio):
    """K distinct experts per token, sampled without replacement with Zipf(s)
    weights over a seeded permutation of the experts (weighted sampling by
    Efraimidis-Spirakis keys u^(1/w), largest K kept, in key order).

    The weights of partition 0's experts are multiplied by a factor alpha,
    found by bisection with the same uniforms u, so that partition 0 receives
    part0_ratio times the mean per-partition load.  Returns (idx, alpha, ratio).
    """
    L = E // P
    perm = perm_rng.permutation(E)
    wz = np.empty(E)
    wz[perm] = 1.0 / np.arange(1, E + 1, dtype=np.float64) ** s
    logu = np.log1p(-rng.random((T, E)))           # log(u), u in (0, 1]
    logu = np.minimum(logu, -1e-300)               # keep strictly negative
    in0 = np.arange(E) < L

    def route(alpha):
        keys = logu / np.where(in0, wz * alpha, wz)    # log of u^(1/w)
        top = np.argpartition(-keys, K - 1, axis=1)[:, :K]
        tk = np.take_along_axis(keys, top, axis=1)
        order = np.argsort(-tk, axis=1, kind="stable")
        return np.take_along_axis(top, order, axis=1).astype(np.int32)

    def load0(alpha):
        return int(np.count_nonzero(route(alpha) < L))

    target = part0_ratio * T * K / P
    lo, hi = -30.0, 30.0                            # log(alpha) bracket
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        if load0(np.exp(mid)) >= target:
            hi = mid
        else:
            lo = mid
    cands = [np.exp(lo), np.exp(hi)]
    alpha = min(cands, key=lambda a: abs(load0(a) - target))
    idx = route(alpha)
    ratio = np.count_nonzero(idx < L) / (T * K / P)
    return idx, float(alpha), float(ratio)


def softmax_weights(rng, idx):
    """fp32 softmax of N(0,1) logits over each token's unmasked entries
    (max subtracted, evaluated in fp64, rounded to fp32); masked entries get 0."""
    T, K = idx.shape
    logits = rng.standard_normal((T, K))
    valid = idx >= 0
    z = np.where(valid, logits, -np.inf)
    m = np.max(z, axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    ez = np.where(valid, np.exp(z - m), 0.0)
    s = ez.sum(axis=1, keepdims=True)
    w = np.where(s > 0, ez / np.where(s > 0, s, 1.0), 0.0)
    return w.astype(np.float32)


def generate(wl: Workload, seed: int | None = None, with_y: bool = True, with_x: bool = True):
    """Inputs for one workload: dict(idx, w, x, y, N, meta).

    idx int32 [T,K] (negative = dropped entry), w fp32 [T,K], x uint16 bf16
    bits [T,H], y uint16 bf16 bits [T*K, H] expert outputs in receive-row
    layout (rows >= N are zero and never read), N = number of valid entries.
    """
    seed = wl.seed if seed is None else seed
    T, H, E, P, K = wl.T, wl.H, wl.E, wl.P, wl.K
    meta = {}
    if wl.routing == "uniform":
        idx = uniform_distinct_routing(_rng(seed, _S_ROUTE), T, E, K)
    elif wl.routing == "zipf":
        idx, alpha, ratio = zipf_routing(_rng(seed, _S_ROUTE), _rng(seed, _S_PERM),
                                         T, E, P, K, wl.zipf_s, wl.part0_ratio)
        meta.update(alpha=alpha, part0_ratio=ratio)
    else:
        raise ValueError(wl.routing)
    if wl.mask_frac > 0 and T > 0:
        n_mask = int(round(wl.mask_frac * T * K))
        pos = _rng(seed, _S_MASK).choice(T * K, n_mask, replace=False)
        idx.reshape(-1)[pos] = -1
    w = softmax_weights(_rng(seed, _S_LOGIT), idx)
    N = int(np.count_nonzero((idx >= 0) & (idx < E)))
    out = dict(idx=np.ascontiguousarray(idx, np.int32), w=w, N=N, meta=meta)
    if with_x:
        rx = _rng(seed, _S_X)
        if wl.outlier_frac > 0 and T > 0:
            x32 = rx.standard_normal((T, H), dtype=np.float32)
            n_out = max(1, int(round(wl.outlier_frac * T)))
            rows = _rng(seed, _S_OUTLIER).choice(T, n_out, replace=False)
            x32[rows] *= np.float32(wl.outlier_scale)
            out["x"] = to_bf16_bits(x32)
            meta["outlier_rows"] = sorted(int(r) for r in rows)
        else:
            out["x"] = _normal_bf16(rx, T, H)
    if with_y:
        y = np.zeros((T * K, H), np.uint16)
        _normal_bf16(_rng(seed, _S_Y), N, H, out=y[:N])
        out["y"] = y
    return out
