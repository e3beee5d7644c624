"""CPU oracle for MoE EP low-latency layout / dispatch / combine.

TEST INFRASTRUCTURE.  Only the tests, the smoke entry point and the bench's
cpu_baseline leg may import this package.  It never imports the product
package and shares no code with it; the arithmetic lives in ep_oracle.c
(plain single-threaded C, fp32 where the method fixes fp32).  This module only
marshals numpy arrays into that library.

Every function here is pinned by CPU tests against things other than itself:
hand-derived values of the OCP E4M3 and bf16 formats, a nearest-value table
encoder, torch's own fp8/bf16 conversions, a stable-sort brute force of the
layout, fp64 error bounds and the identity-expert round trip.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None
_lib_path = None


def use_library(path=None):
    """Load the oracle from another build of ep_oracle.c (tests that plant a
    mistake in a copy of the oracle use this); None restores the default."""
    global _lib, _lib_path
    _lib, _lib_path = None, path


def lib():
    global _lib
    if _lib is None:
        path = _lib_path or _build.LIB
        if _lib_path is None and not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int, ctypes.c_int64
        L.oracle_layout.argtypes = [P, i32, i32, i32, i32, P, P, P, P, P, P, P]
        L.oracle_layout.restype = i32
        L.oracle_dispatch_fp8_range.argtypes = [P, i32, i32, i32, P, i32, i32, P, P]
        L.oracle_dispatch_fp8_range.restype = i32
        L.oracle_dispatch_bf16.argtypes = [P, i32, i32, i32, P, P]
        L.oracle_dispatch_bf16.restype = i32
        L.oracle_combine_range.argtypes = [P, P, P, i32, i32, i32, i32, i32, P]
        L.oracle_combine_range.restype = i32
        L.oracle_e4m3fn_encode_array.argtypes = [P, i64, P]
        L.oracle_e4m3fn_encode_array.restype = None
        L.oracle_bf16_rne_array.argtypes = [P, i64, P]
        L.oracle_bf16_rne_array.restype = None
        L.oracle_dedup_layout.argtypes = [P, i32, i32, i32, i32, P, P, P, P, P, P]
        L.oracle_dedup_layout.restype = i32
        L.oracle_combine_partial.argtypes = [P, P, P, P, P, i32, i32, i32, i32, P]
        L.oracle_combine_partial.restype = i32
        L.oracle_combine_reduce.argtypes = [P, P, i32, i32, i32, P]
        L.oracle_combine_reduce.restype = i32
        L.oracle_e4m3fn_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3fn_decode.restype = ctypes.c_float
        _lib = L
    return _lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError("expected %s, got %s" % (dtype, a.dtype))
    return a


class OracleError(ValueError):
    pass


def layout(topk_idx, E, P):
    """Counts, scans and deterministic slots; returns a dict of int32/uint32 arrays."""
    idx = _c(topk_idx, np.int32)
    T, K = idx.shape
    n = T * K
    out = dict(
        expert_count=np.zeros(E, np.int32),
        expert_offset=np.zeros(E + 1, np.int32),
        part_count=np.zeros(P, np.int32),
        part_offset=np.zeros(P + 1, np.int32),
        row_of_pair=np.zeros(n, np.int32),
        src_pair=np.zeros(n, np.int32),
        status=np.zeros(1, np.uint32),
    )
    rc = lib().oracle_layout(_ptr(idx), T, K, E, P,
                             *[_ptr(out[k]) for k in ("expert_count", "expert_offset", "part_count",
                                                      "part_offset", "row_of_pair", "src_pair", "status")])
    if rc != 0:
        raise OracleError("oracle_layout rejected T=%d K=%d E=%d P=%d" % (T, K, E, P))
    return out


def dispatch_fp8(x_bf16, row_of_pair, K, rows=None, t0=0, t1=None, recv_x=None, recv_scales=None):
    """fp8 e4m3fn dispatch with per-128-column fp32 scales.

    x_bf16: uint16 [T, H]; row_of_pair: int32 [T*K].  Returns (recv_x uint8 [rows, H],
    recv_scales float32 [rows, H/128]); untouched rows are left as given (zeros if the
    buffers are created here).
    """
    x = _c(x_bf16, np.uint16)
    T, H = x.shape
    rop = _c(row_of_pair, np.int32).reshape(-1)
    rows = T * K if rows is None else rows
    t1 = T if t1 is None else t1
    if recv_x is None:
        recv_x = np.zeros((rows, H), np.uint8)
    if recv_scales is None:
        recv_scales = np.zeros((rows, H // 128), np.float32)
    rc = lib().oracle_dispatch_fp8_range(_ptr(x), T, H, K, _ptr(rop), t0, t1,
                                         _ptr(recv_x), _ptr(recv_scales))
    if rc != 0:
        raise OracleError("oracle_dispatch_fp8 rejected T=%d H=%d K=%d" % (T, H, K))
    return recv_x, recv_scales


def dispatch_bf16(x_bf16, row_of_pair, K, rows=None, recv_x=None):
    x = _c(x_bf16, np.uint16)
    T, H = x.shape
    rop = _c(row_of_pair, np.int32).reshape(-1)
    rows = T * K if rows is None else rows
    if recv_x is None:
        recv_x = np.zeros((rows, H), np.uint16)
    rc = lib().oracle_dispatch_bf16(_ptr(x), T, H, K, _ptr(rop), _ptr(recv_x))
    if rc != 0:
        raise OracleError("oracle_dispatch_bf16 rejected T=%d H=%d K=%d" % (T, H, K))
    return recv_x


def combine(y_bf16, row_of_pair, topk_w, T, H, K, t0=0, t1=None):
    """Gather-reduce in fp32 (fmaf, fixed k order) -> bf16 (uint16 [t1-t0, H])."""
    y = _c(y_bf16, np.uint16)
    rop = _c(row_of_pair, np.int32).reshape(-1)
    w = _c(topk_w, np.float32).reshape(-1)
    t1 = T if t1 is None else t1
    out = np.zeros((T, H), np.uint16)
    rc = lib().oracle_combine_range(_ptr(y), _ptr(rop), _ptr(w), T, H, K, t0, t1, _ptr(out))
    if rc != 0:
        raise OracleError("oracle_combine rejected T=%d H=%d K=%d" % (T, H, K))
    return out[t0:t1]


def e4m3fn_encode(values_f32):
    v = _c(values_f32, np.float32).reshape(-1)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_e4m3fn_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def e4m3fn_decode(code):
    return float(lib().oracle_e4m3fn_decode(int(code)))


def bf16_rne(values_f32):
    v = _c(values_f32, np.float32).reshape(-1)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_bf16_rne_array(_ptr(v), v.size, _ptr(out))
    return out


def dedup_layout(topk_idx, E, P):
    """Per-destination deduplicated layout (one row per (token, partition))."""
    idx = _c(topk_idx, np.int32)
    T, K = idx.shape
    out = dict(tp_row=np.zeros(T * P, np.int32), part_tokens=np.zeros(P, np.int32),
               part_token_offset=np.zeros(P + 1, np.int32), tp_src=np.zeros(T * P, np.int32),
               kmask=np.zeros(T * P, np.uint32), status=np.zeros(1, np.uint32))
    rc = lib().oracle_dedup_layout(_ptr(idx), T, K, E, P,
                                   *[_ptr(out[k]) for k in ("tp_row", "part_tokens", "part_token_offset",
                                                            "tp_src", "kmask", "status")])
    if rc != 0:
        raise OracleError("oracle_dedup_layout rejected T=%d K=%d E=%d P=%d" % (T, K, E, P))
    return out


def combine_partial(y_bf16, row_of_pair, topk_w, tp_row, kmask, T, H, K, P, rows=None):
    """Level 1 of the two-level combine: bf16 partial per (token, partition) row."""
    y = _c(y_bf16, np.uint16)
    rop = _c(row_of_pair, np.int32).reshape(-1)
    w = _c(topk_w, np.float32).reshape(-1)
    tr = _c(tp_row, np.int32).reshape(-1)
    km = _c(kmask, np.uint32).reshape(-1)
    rows = T * P if rows is None else rows
    part = np.zeros((rows, H), np.uint16)
    rc = lib().oracle_combine_partial(_ptr(y), _ptr(rop), _ptr(w), _ptr(tr), _ptr(km), T, H, K, P,
                                      _ptr(part))
    if rc != 0:
        raise OracleError("oracle_combine_partial rejected")
    return part


def combine_reduce(partial_bf16, tp_row, T, H, P):
    """Level 2: fp32 sum of a token's partials in partition order -> bf16."""
    part = _c(partial_bf16, np.uint16)
    tr = _c(tp_row, np.int32).reshape(-1)
    out = np.zeros((T, H), np.uint16)
    rc = lib().oracle_combine_reduce(_ptr(part), _ptr(tr), T, H, P, _ptr(out))
    if rc != 0:
        raise OracleError("oracle_combine_reduce rejected")
    return out
