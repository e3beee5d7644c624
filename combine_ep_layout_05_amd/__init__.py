"""MI355X (gfx950) MoE expert-parallel low-latency layout / dispatch / combine.

Thin ctypes binding of libep_mi355x.so (declared in include/ep.h).  The
functions keep the C names; they only check tensor dtypes/devices, pass raw
device pointers and torch's current stream, and turn a negative return code
into an exception.  Every step of the path runs in the library's HIP kernels;
there is no fallback: if the library is not built, importing the package
raises.

    from combine_ep_layout_05_amd import EpBuffers
    buf = EpBuffers(T, H, K, E, P, payload="fp8")     # persistent outputs
    buf.layout(topk_idx_i32)                            # counts, offsets, slots
    buf.dispatch(x_bf16)                                # -> buf.recv_x, buf.recv_scales
    out = buf.combine(expert_out_bf16, topk_w_f32)      # -> bf16 [T, H]
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libep_mi355x.so")

EP_OK, EP_EINVAL, EP_ENOTSUP, EP_EHIP, EP_ESCRATCH = 0, -1, -2, -3, -4
EP_NOALLOC_SCRATCH_BYTES = 4 << 20
EP_PAYLOAD_FP8_E4M3FN, EP_PAYLOAD_BF16 = 0, 1
EP_STATUS_BAD_EXPERT_ID = 1
PAYLOADS = {"fp8": EP_PAYLOAD_FP8_E4M3FN, "bf16": EP_PAYLOAD_BF16}

if not os.path.exists(LIB_PATH):
    raise ImportError("libep_mi355x.so is not built: run combine_ep_layout_05_amd/build.py "
                      "(or __graft_entry__.build()) first")

_lib = ctypes.CDLL(LIB_PATH)
_P, _I, _I64, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
_SIGS = {
    "ep_layout_workspace_bytes": ([_I, _I, _I], _SZ),
    "ep_layout": ([_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], _I),
    "ep_dispatch": ([_P, _I, _I, _I, _P, _I, _P, _P, _P], _I),
    "ep_combine": ([_P, _P, _P, _I, _I, _I, _P, _P], _I),
    "ep_layout_dispatch": ([_P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _SZ,
                            _P, _P, _P], _I),
    "ep_layout_dispatch_geom": ([_P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P,
                                 _SZ, _P, _P, _I, _I, _I, _P], _I),
    "ep_layout_dispatch_plan": ([_I, _I, _I, _I, _I, _I, _I, _I, _I, _P], _I),
    "ep_layout_dispatch_noalloc": ([_P, _P, _I, _I, _I, _I, _I, _I] + [_P] * 10, _I),
    "ep_graph_begin": ([_P], _I),
    "ep_graph_end": ([_P, ctypes.POINTER(_P)], _I),
    "ep_graph_launch": ([_P, _P], _I),
    "ep_graph_destroy": ([_P], _I),
    "ep_e4m3fn_encode": ([_P, _I64, _P, _P], _I),
    "ep_topk_idx_narrow": ([_P, _I64, _P, _P], _I),
    "ep_dispatch_geom": ([_P, _I, _I, _I, _P, _I, _P, _P, _I, _I, _I, _P], _I),
    "ep_combine_geom": ([_P, _P, _P, _I, _I, _I, _P, _I, _I, _I, _P], _I),
    "ep_combine_plan": ([_I, _I, _I, _I, _I, _I, _P], _I),
    "ep_dedup_layout_workspace_bytes": ([_I, _I, _I, _I], _SZ),
    "ep_dedup_layout": ([_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], _I),
    "ep_combine_partial": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P], _I),
    "ep_dedup_layout_dispatch_workspace_bytes": ([_I, _I, _I, _I], _SZ),
    "ep_dedup_layout_dispatch": ([_P, _P, _I, _I, _I, _I, _I, _I] + [_P] * 12 + [_P, _SZ, _P, _P, _P],
                                 _I),
    "ep_dedup_layout_dispatch_geom": ([_P, _P, _I, _I, _I, _I, _I, _I] + [_P] * 12
                                      + [_P, _SZ, _P, _P, _I, _I, _I, _P], _I),
    "ep_dedup_layout_dispatch_plan": ([_I, _I, _I, _I, _I, _I, _I, _I, _I, _P], _I),
    "ep_combine_reduce": ([_P, _P, _I, _I, _I, _P, _P], _I),
    "ep_strerror": ([_I], ctypes.c_char_p),
    "ep_last_hip_error": ([], _I),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes, _f.restype = _args, _res

PLAN_KINDS = {0: "fused_tiny", 1: "fused_count", 2: "fused_general", 3: "layout_then_dispatch"}


class EpError(RuntimeError):
    def __init__(self, fn, code):
        msg = _lib.ep_strerror(code).decode()
        if code == EP_EHIP:
            msg += " (hipError %d)" % _lib.ep_last_hip_error()
        super().__init__("%s: %s" % (fn, msg))
        self.code = code


def _check(fn, code):
    if code != EP_OK:
        raise EpError(fn, code)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device tensor expected, got a %s tensor" % t.device)
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return ctypes.c_void_p(t.data_ptr())


def _dt(t, *dtypes):
    if t is not None and t.dtype not in dtypes:
        raise TypeError("dtype %s not in %s" % (t.dtype, dtypes))


# Shape checks, made before any pointer reaches the library: a tensor smaller
# than the call assumes would be read or written past its end on the device.
def _numel(t, n, name):
    if t is None or t.numel() != n:
        raise ValueError("%s: expected %d elements, got %s" % (name, n, None if t is None else t.numel()))


def _rows(t, min_rows, width, name):
    if t is None or t.dim() != 2 or t.shape[0] < min_rows or t.shape[1] != width:
        raise ValueError("%s: expected a 2-D tensor of at least %d rows and %d columns, got %s" % (
            name, min_rows, width, None if t is None else tuple(t.shape)))


def _matrix(t, shape, name):
    if t is None or tuple(t.shape) != tuple(shape):
        raise ValueError("%s: expected shape %s, got %s" % (name, tuple(shape),
                                                             None if t is None else tuple(t.shape)))


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_U32 = (torch.int32, torch.uint32)


def _layout_outputs(T, K, E, P, expert_count, expert_offset, part_count, part_offset, row_of_pair,
                    src_pair, status):
    for t in (expert_count, expert_offset, part_count, part_offset, row_of_pair, src_pair):
        _dt(t, torch.int32)
    _dt(status, *_U32)
    _numel(expert_count, E, "expert_count")
    _numel(expert_offset, E + 1, "expert_offset")
    _numel(part_count, P, "part_count")
    _numel(part_offset, P + 1, "part_offset")
    _numel(row_of_pair, T * K, "row_of_pair")
    _numel(src_pair, T * K, "src_pair")
    if status is None or status.numel() < 1:
        raise ValueError("status: one element expected")


def _receive(payload, rows, H, recv_x, recv_scales):
    """recv_x / recv_scales for `rows` receive rows of hidden size H."""
    if payload == EP_PAYLOAD_FP8_E4M3FN:
        _dt(recv_x, torch.uint8)
        _dt(recv_scales, torch.float32)
        _rows(recv_x, rows, H, "recv_x (fp8 bytes)")
        _rows(recv_scales, rows, H // 128, "recv_scales")
    elif payload == EP_PAYLOAD_BF16:
        _dt(recv_x, *_BF16)
        _rows(recv_x, rows, H, "recv_x (bf16)")


def _ws_bytes(ws):
    return 0 if ws is None else ws.numel() * ws.element_size()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _geometry(geometry):
    """(waves_per_block, max_blocks[, slice_cols]) -> three ints."""
    g = tuple(int(v) for v in geometry)
    if len(g) == 2:
        g = g + (0,)
    if len(g) != 3:
        raise ValueError("geometry: (waves_per_block, max_blocks[, slice_cols]) expected")
    return g


def library_path() -> str:
    return LIB_PATH


def ep_layout_workspace_bytes(T: int, K: int, E: int) -> int:
    return int(_lib.ep_layout_workspace_bytes(T, K, E))


def ep_layout(topk_idx, E, P, expert_count, expert_offset, part_count, part_offset,
              row_of_pair, src_pair, status, ws=None, stream=None):
    """topk_idx int32 [T, K] -> the layout outputs (see include/ep.h)."""
    _dt(topk_idx, torch.int32)
    T, K = topk_idx.shape
    _layout_outputs(T, K, E, P, expert_count, expert_offset, part_count, part_offset, row_of_pair,
                    src_pair, status)
    _check("ep_layout", _lib.ep_layout(
        _ptr(topk_idx), T, K, E, P, _ptr(expert_count), _ptr(expert_offset), _ptr(part_count),
        _ptr(part_offset), _ptr(row_of_pair), _ptr(src_pair), _ptr(status), _ptr(ws), _ws_bytes(ws),
        _stream(stream)))


def ep_dispatch(x, K, row_of_pair, payload, recv_x, recv_scales=None, stream=None, geometry=None):
    """x bf16 [T, H] -> recv_x (uint8 fp8 bytes or bf16) [T*K, H], recv_scales fp32 [T*K, H/128].
    geometry: None (library default) or (waves_per_block, max_blocks[, slice_cols])."""
    _dt(x, *_BF16)
    _dt(row_of_pair, torch.int32)
    payload = PAYLOADS.get(payload, payload)
    T, H = x.shape
    _numel(row_of_pair, T * K, "row_of_pair")
    _receive(payload, T * K, H, recv_x, recv_scales)
    if geometry is None:
        _check("ep_dispatch", _lib.ep_dispatch(_ptr(x), T, H, K, _ptr(row_of_pair), payload,
                                               _ptr(recv_x), _ptr(recv_scales), _stream(stream)))
    else:
        wv, mb, sc = _geometry(geometry)
        _check("ep_dispatch_geom", _lib.ep_dispatch_geom(
            _ptr(x), T, H, K, _ptr(row_of_pair), payload, _ptr(recv_x), _ptr(recv_scales), wv, mb,
            sc, _stream(stream)))


def ep_layout_dispatch(topk_idx, x, E, P, payload, expert_count, expert_offset, part_count,
                       part_offset, row_of_pair, src_pair, status, ws, recv_x, recv_scales=None,
                       stream=None, geometry=None):
    """ep_layout followed by ep_dispatch, as one launch for small batches.
    geometry: None (the library's choice) or (waves_per_block, max_blocks[,
    slice_cols]) as ep_layout_dispatch_geom takes it."""
    _dt(topk_idx, torch.int32)
    _dt(x, *_BF16)
    payload = PAYLOADS.get(payload, payload)
    T, K = topk_idx.shape
    if x.dim() != 2 or x.shape[0] != T:
        raise ValueError("x: expected [%d, H], got %s" % (T, tuple(x.shape)))
    H = x.shape[1]
    _layout_outputs(T, K, E, P, expert_count, expert_offset, part_count, part_offset, row_of_pair,
                    src_pair, status)
    _receive(payload, T * K, H, recv_x, recv_scales)
    args = (_ptr(topk_idx), _ptr(x), T, H, K, E, P, payload, _ptr(expert_count),
            _ptr(expert_offset), _ptr(part_count), _ptr(part_offset), _ptr(row_of_pair),
            _ptr(src_pair), _ptr(status), _ptr(ws), _ws_bytes(ws), _ptr(recv_x), _ptr(recv_scales))
    if geometry is None:
        _check("ep_layout_dispatch", _lib.ep_layout_dispatch(*args, _stream(stream)))
    else:
        _check("ep_layout_dispatch_geom",
               _lib.ep_layout_dispatch_geom(*args, *_geometry(geometry), _stream(stream)))


def _plan(name, T, H, K, E, P, payload, geometry):
    payload = PAYLOADS.get(payload, payload)
    plan = (ctypes.c_int32 * 4)()
    wv, mb, sc = _geometry(geometry) if geometry is not None else (0, 0, 0)
    _check(name, getattr(_lib, name)(T, H, K, E, P, payload, wv, mb, sc,
                                     ctypes.cast(plan, ctypes.c_void_p)))
    kind = PLAN_KINDS[plan[0]]
    d = {"kernel": kind, "waves": int(plan[1]), "slice_cols": int(plan[3])}
    d["max_blocks" if kind == "layout_then_dispatch" else "blocks"] = int(plan[2])
    return d


def ep_dedup_layout_dispatch_plan(T, H, K, E, P, payload, geometry=None):
    """How ep_dedup_layout_dispatch(_geom) would run this batch (host only),
    in the form ep_layout_dispatch_plan returns."""
    return _plan("ep_dedup_layout_dispatch_plan", T, H, K, E, P, payload, geometry)


def ep_layout_dispatch_plan(T, H, K, E, P, payload, geometry=None):
    """How ep_layout_dispatch(_geom) would run this batch (host only):
    {"kernel": ..., "waves": ..., "blocks" or "max_blocks": ..., "slice_cols": ...}."""
    return _plan("ep_layout_dispatch_plan", T, H, K, E, P, payload, geometry)


def ep_combine_plan(T, H, K, geometry=None):
    """The geometry ep_combine (geometry None) or ep_combine_geom would launch
    a combine of T tokens x top-k K at hidden size H with (host only):
    {"waves": ..., "max_blocks": ..., "slice_cols": ..., "streaming": bool}."""
    plan = (ctypes.c_int32 * 4)()
    wv, mb, sc = _geometry(geometry) if geometry is not None else (0, 0, 0)
    _check("ep_combine_plan", _lib.ep_combine_plan(T, H, K, wv, mb, sc,
                                                   ctypes.cast(plan, ctypes.c_void_p)))
    return {"waves": int(plan[0]), "max_blocks": int(plan[1]), "slice_cols": int(plan[2]),
            "streaming": bool(plan[3])}


def ep_layout_dispatch_noalloc(topk_idx, x, E, P, payload, expert_count, expert_offset,
                               part_count, part_offset, row_of_pair, src_pair, status, recv_x,
                               recv_scales=None, stream=None):
    """ep_layout_dispatch with the library's own per-device scratch buffer as
    the layout workspace: the call allocates nothing (see include/ep.h)."""
    _dt(topk_idx, torch.int32)
    _dt(x, *_BF16)
    payload = PAYLOADS.get(payload, payload)
    T, K = topk_idx.shape
    if x.dim() != 2 or x.shape[0] != T:
        raise ValueError("x: expected [%d, H], got %s" % (T, tuple(x.shape)))
    H = x.shape[1]
    _layout_outputs(T, K, E, P, expert_count, expert_offset, part_count, part_offset, row_of_pair,
                    src_pair, status)
    _receive(payload, T * K, H, recv_x, recv_scales)
    _check("ep_layout_dispatch_noalloc", _lib.ep_layout_dispatch_noalloc(
        _ptr(topk_idx), _ptr(x), T, H, K, E, P, payload, _ptr(expert_count), _ptr(expert_offset),
        _ptr(part_count), _ptr(part_offset), _ptr(row_of_pair), _ptr(src_pair), _ptr(status),
        _ptr(recv_x), _ptr(recv_scales), _stream(stream)))


def ep_combine(expert_out, row_of_pair, topk_w, out, stream=None, geometry=None):
    """expert_out bf16 [T*K, H] (receive-row layout), topk_w fp32 [T, K] -> out bf16 [T, H].
    geometry: None (library default) or (waves_per_block, max_blocks[, slice_cols])."""
    _dt(expert_out, *_BF16)
    _dt(out, *_BF16)
    _dt(topk_w, torch.float32)
    _dt(row_of_pair, torch.int32)
    T, K = topk_w.shape
    if out.dim() != 2 or out.shape[0] != T:
        raise ValueError("out: expected [%d, H], got %s" % (T, tuple(out.shape)))
    H = out.shape[1]
    _numel(row_of_pair, T * K, "row_of_pair")
    _rows(expert_out, T * K, H, "expert_out")
    if geometry is None:
        _check("ep_combine", _lib.ep_combine(_ptr(expert_out), _ptr(row_of_pair), _ptr(topk_w), T,
                                             H, K, _ptr(out), _stream(stream)))
    else:
        wv, mb, sc = _geometry(geometry)
        _check("ep_combine_geom", _lib.ep_combine_geom(
            _ptr(expert_out), _ptr(row_of_pair), _ptr(topk_w), T, H, K, _ptr(out), wv, mb, sc,
            _stream(stream)))


def ep_topk_idx_narrow(topk_idx64, out_i32, stream=None):
    """int64 expert ids -> int32 ids on the GPU (negative -> -1, above
    INT32_MAX -> INT32_MAX); out_i32 must have as many elements."""
    _dt(topk_idx64, torch.int64)
    _dt(out_i32, torch.int32)
    _numel(out_i32, topk_idx64.numel(), "out_i32")
    _check("ep_topk_idx_narrow", _lib.ep_topk_idx_narrow(_ptr(topk_idx64), topk_idx64.numel(),
                                                         _ptr(out_i32), _stream(stream)))


def _tokens(buf, topk_idx):
    """The batch's token count, at most the buffers' T, from topk_idx [n, K]."""
    if topk_idx.dim() != 2 or topk_idx.shape[1] != buf.K or topk_idx.shape[0] > buf.T:
        raise ValueError("topk_idx: expected [n, %d] with n <= %d, got %s" % (
            buf.K, buf.T, tuple(topk_idx.shape)))
    return topk_idx.shape[0]


def _ids32(buf, topk_idx, stream):
    """topk_idx as the int32 ids the layouts take: int32 as given, int64
    narrowed into the buffers' own int32 ids (one extra launch)."""
    if topk_idx.dtype != torch.int64:
        return topk_idx
    n = _tokens(buf, topk_idx)
    ep_topk_idx_narrow(topk_idx, buf.idx32[:n], stream)
    return buf.idx32[:n]


def _same_tokens(buf, n, what):
    if n != buf.n:
        raise ValueError("%s: %d tokens, but the last layout was of %d" % (what, n, buf.n))


def ep_e4m3fn_encode(values_f32, out_u8, stream=None):
    _dt(values_f32, torch.float32)
    _dt(out_u8, torch.uint8)
    _numel(out_u8, values_f32.numel(), "out_u8")
    _check("ep_e4m3fn_encode", _lib.ep_e4m3fn_encode(_ptr(values_f32), values_f32.numel(),
                                                     _ptr(out_u8), _stream(stream)))


def ep_dedup_layout_workspace_bytes(T: int, K: int, E: int, P: int) -> int:
    return int(_lib.ep_dedup_layout_workspace_bytes(T, K, E, P))


def _dedup_outputs(T, P, tp_row, part_tokens, part_token_offset, tp_src, kmask, status):
    for t in (tp_row, part_tokens, part_token_offset, tp_src):
        _dt(t, torch.int32)
    _dt(kmask, *_U32)
    _dt(status, *_U32)
    _numel(tp_row, T * P, "tp_row")
    _numel(part_tokens, P, "part_tokens")
    _numel(part_token_offset, P + 1, "part_token_offset")
    _numel(tp_src, T * P, "tp_src")
    _numel(kmask, T * P, "kmask")
    if status is None or status.numel() < 1:
        raise ValueError("status: one element expected")


def ep_dedup_layout(topk_idx, E, P, tp_row, part_tokens, part_token_offset, tp_src, kmask,
                    status, ws=None, stream=None):
    """topk_idx int32 [T, K] -> per-destination (dedup) layout (see include/ep.h)."""
    _dt(topk_idx, torch.int32)
    T, K = topk_idx.shape
    _dedup_outputs(T, P, tp_row, part_tokens, part_token_offset, tp_src, kmask, status)
    _check("ep_dedup_layout", _lib.ep_dedup_layout(
        _ptr(topk_idx), T, K, E, P, _ptr(tp_row), _ptr(part_tokens), _ptr(part_token_offset),
        _ptr(tp_src), _ptr(kmask), _ptr(status), _ptr(ws), _ws_bytes(ws), _stream(stream)))


def ep_dedup_layout_dispatch_workspace_bytes(T: int, K: int, E: int, P: int) -> int:
    return int(_lib.ep_dedup_layout_dispatch_workspace_bytes(T, K, E, P))


def ep_dedup_layout_dispatch(topk_idx, x, E, P, payload, expert_count, expert_offset, part_count,
                             part_offset, row_of_pair, src_pair, tp_row, part_tokens,
                             part_token_offset, tp_src, kmask, status, ws, recv_x,
                             recv_scales=None, stream=None, geometry=None):
    """Per-expert layout + dedup layout + dedup dispatch (one launch for small
    batches).  geometry: None (the library's choice) or (waves_per_block,
    max_blocks[, slice_cols]) as ep_dedup_layout_dispatch_geom takes it."""
    _dt(topk_idx, torch.int32)
    _dt(x, *_BF16)
    payload = PAYLOADS.get(payload, payload)
    T, K = topk_idx.shape
    if x.dim() != 2 or x.shape[0] != T:
        raise ValueError("x: expected [%d, H], got %s" % (T, tuple(x.shape)))
    H = x.shape[1]
    _layout_outputs(T, K, E, P, expert_count, expert_offset, part_count, part_offset, row_of_pair,
                    src_pair, status)
    _dedup_outputs(T, P, tp_row, part_tokens, part_token_offset, tp_src, kmask, status)
    _receive(payload, T * P, H, recv_x, recv_scales)
    args = (_ptr(topk_idx), _ptr(x), T, H, K, E, P, payload, _ptr(expert_count),
            _ptr(expert_offset), _ptr(part_count), _ptr(part_offset), _ptr(row_of_pair),
            _ptr(src_pair), _ptr(tp_row), _ptr(part_tokens), _ptr(part_token_offset), _ptr(tp_src),
            _ptr(kmask), _ptr(status), _ptr(ws), _ws_bytes(ws), _ptr(recv_x), _ptr(recv_scales))
    if geometry is None:
        _check("ep_dedup_layout_dispatch", _lib.ep_dedup_layout_dispatch(*args, _stream(stream)))
    else:
        _check("ep_dedup_layout_dispatch_geom",
               _lib.ep_dedup_layout_dispatch_geom(*args, *_geometry(geometry), _stream(stream)))


def ep_combine_partial(expert_out, row_of_pair, topk_w, tp_row, kmask, P, partial, stream=None):
    """Level 1: expert_out bf16 [T*K, H] -> partial bf16 [T*P, H] (rows of present couples)."""
    _dt(expert_out, *_BF16)
    _dt(partial, *_BF16)
    _dt(topk_w, torch.float32)
    _dt(row_of_pair, torch.int32)
    _dt(tp_row, torch.int32)
    _dt(kmask, *_U32)
    T, K = topk_w.shape
    if partial.dim() != 2:
        raise ValueError("partial: a 2-D tensor expected")
    H = partial.shape[1]
    _rows(partial, T * P, H, "partial")
    _rows(expert_out, T * K, H, "expert_out")
    _numel(row_of_pair, T * K, "row_of_pair")
    _numel(tp_row, T * P, "tp_row")
    _numel(kmask, T * P, "kmask")
    _check("ep_combine_partial", _lib.ep_combine_partial(
        _ptr(expert_out), _ptr(row_of_pair), _ptr(topk_w), _ptr(tp_row), _ptr(kmask), T, H, K, P,
        _ptr(partial), _stream(stream)))


def ep_combine_reduce(partial, tp_row, T, P, out, stream=None):
    """Level 2: partial bf16 [T*P, H] -> out bf16 [T, H] (partition-order fp32 sum)."""
    _dt(partial, *_BF16)
    _dt(out, *_BF16)
    _dt(tp_row, torch.int32)
    if out.dim() != 2 or out.shape[0] != T:
        raise ValueError("out: expected [%d, H], got %s" % (T, tuple(out.shape)))
    H = out.shape[1]
    _rows(partial, T * P, H, "partial")
    _numel(tp_row, T * P, "tp_row")
    _check("ep_combine_reduce", _lib.ep_combine_reduce(_ptr(partial), _ptr(tp_row), T, H, P,
                                                       _ptr(out), _stream(stream)))


class EpGraph:
    """A recorded sequence of ep_* calls (HIP graph), replayed with ep_graph_launch."""

    def __init__(self, handle):
        self._h = ctypes.c_void_p(handle)

    def launch(self, stream=None):
        _check("ep_graph_launch", _lib.ep_graph_launch(self._h, _stream(stream)))

    def bind(self, stream=None):
        """A zero-argument callable that replays the graph on `stream` (torch's
        current stream when None, looked up now): the handle and the stream
        are marshalled once, as a serving loop that replays one graph per
        step would do.  Each call still checks the return code."""
        f, h, s = _lib.ep_graph_launch, self._h, _stream(stream)

        def replay():
            rc = f(h, s)
            if rc != 0:
                _check("ep_graph_launch", rc)
        return replay

    def destroy(self):
        if self._h:
            _check("ep_graph_destroy", _lib.ep_graph_destroy(self._h))
            self._h = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def ep_graph_begin(stream):
    _check("ep_graph_begin", _lib.ep_graph_begin(_stream(stream)))


def ep_graph_end(stream) -> EpGraph:
    h = ctypes.c_void_p()
    _check("ep_graph_end", _lib.ep_graph_end(_stream(stream), ctypes.byref(h)))
    return EpGraph(h.value)


class EpBuffers:
    """Persistent device buffers for one shape (allocated once, reused by every
    call, so the calls can be captured into a graph).  T is the most tokens a
    batch may hold: a layout of n <= T tokens (topk_idx [n, K]) sets the batch
    size the dispatch and the combine after it work on, over the first rows
    of the same buffers (so a graph may still capture them)."""

    def __init__(self, T, H, K, E, P, payload="fp8", device="cuda", geometry=None):
        """geometry: None (library defaults), "tuned" (the saved rules for this
        shape, where there are any) or a dict with any of the keys
        "layout_dispatch", "dispatch", "combine", each (waves_per_block,
        max_blocks, slice_cols) as the *_geom entry points take it."""
        self.T, self.H, self.K, self.E, self.P = T, H, K, E, P
        self.n = T                                        # tokens of the current batch
        self.payload = payload
        if geometry == "tuned":
            from . import tuning
            geometry = {ph: tuning.lookup(ph, T, H, K, payload)
                        for ph in ("layout_dispatch", "dispatch", "combine")}
        self.geometry = {k: _geometry(v) for k, v in (geometry or {}).items() if v is not None}
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.expert_count = torch.empty(E, **i32)
        self.expert_offset = torch.empty(E + 1, **i32)
        self.part_count = torch.empty(P, **i32)
        self.part_offset = torch.empty(P + 1, **i32)
        self.row_of_pair = torch.empty(T * K, **i32)
        self.src_pair = torch.empty(T * K, **i32)
        self.status = torch.empty(1, **i32)
        self.idx32 = torch.empty((T, K), **i32)          # int64 ids narrowed here
        wsb = ep_layout_workspace_bytes(T, K, E)
        self.ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
        if payload == "fp8":
            self.recv_x = torch.empty((T * K, H), dtype=torch.uint8, device=dev)
            self.recv_scales = torch.empty((T * K, H // 128), dtype=torch.float32, device=dev)
        else:
            self.recv_x = torch.empty((T * K, H), dtype=torch.bfloat16, device=dev)
            self.recv_scales = None
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

    def _views(self, n):
        m = n * self.K
        return (self.row_of_pair[:m], self.src_pair[:m], self.recv_x[:m],
                None if self.recv_scales is None else self.recv_scales[:m])

    def layout(self, topk_idx, stream=None):
        """topk_idx int32 [n, K], n <= T, or int64 (narrowed first, one extra
        launch); sets the batch to n tokens."""
        n = _tokens(self, topk_idx)
        topk_idx = _ids32(self, topk_idx, stream)
        rop, src, _, _ = self._views(n)
        ep_layout(topk_idx, self.E, self.P, self.expert_count, self.expert_offset, self.part_count,
                  self.part_offset, rop, src, self.status, self.ws, stream)
        self.n = n

    def layout_dispatch(self, topk_idx, x, stream=None):
        """topk_idx int32 [n, K], n <= T, or int64 (narrowed first, one extra
        launch), x bf16 [n, H]; sets the batch to n tokens."""
        n = _tokens(self, topk_idx)
        topk_idx = _ids32(self, topk_idx, stream)
        rop, src, rx, rs = self._views(n)
        ep_layout_dispatch(topk_idx, x, self.E, self.P, self.payload, self.expert_count,
                           self.expert_offset, self.part_count, self.part_offset, rop, src,
                           self.status, self.ws, rx, rs, stream, self.geometry.get("layout_dispatch"))
        self.n = n

    def plan(self):
        """What layout_dispatch launches for this shape and geometry, and the
        dispatch / combine geometry (host only)."""
        d = {"layout_dispatch": ep_layout_dispatch_plan(self.T, self.H, self.K, self.E, self.P,
                                                        self.payload,
                                                        self.geometry.get("layout_dispatch"))}
        g = self.geometry.get("dispatch")
        d["dispatch"] = "library default (4 waves, uncapped, 512 columns)" if g is None else \
            {"waves": g[0], "max_blocks": g[1], "slice_cols": g[2] or 512}
        g = self.geometry.get("combine")
        c = ep_combine_plan(self.T, self.H, self.K, g)
        d["combine"] = dict(c, source="library default" if g is None else "given")
        return d

    def dispatch(self, x, stream=None):
        """x bf16 [n, H] of the current batch (the last layout's n tokens)."""
        _same_tokens(self, x.shape[0], "x")
        rop, _, rx, rs = self._views(self.n)
        ep_dispatch(x, self.K, rop, self.payload, rx, rs, stream, self.geometry.get("dispatch"))

    def combine(self, expert_out, topk_w, stream=None):
        """expert_out bf16 [>= n*K, H], topk_w fp32 [n, K] of the current batch;
        returns out[:n]."""
        _same_tokens(self, topk_w.shape[0], "topk_w")
        rop, _, _, _ = self._views(self.n)
        out = self.out[:self.n]
        ep_combine(expert_out, rop, topk_w, out, stream, self.geometry.get("combine"))
        return out


class EpDedupBuffers:
    """Persistent device buffers of the per-destination (dedup) path for one
    shape: the dedup layout, the dedup receive rows (one per present (token,
    partition) couple), the partial rows and the output.  T is the most tokens
    a batch may hold; a layout of n <= T tokens sets the batch size, as in
    EpBuffers."""

    def __init__(self, T, H, K, E, P, payload="fp8", device="cuda", geometry=None):
        """geometry: None (the library's choice), "tuned" (the saved rule of
        the dedup_layout_dispatch phase for this shape, if any) or a
        (waves_per_block, max_blocks[, slice_cols]) tuple, used by
        layout_dispatch when it is given none."""
        self.T, self.H, self.K, self.E, self.P = T, H, K, E, P
        self.n = T                                        # tokens of the current batch
        self.payload = payload
        if geometry == "tuned":
            from . import tuning
            geometry = tuning.lookup("dedup_layout_dispatch", T, H, K, payload)
        self.geometry = None if geometry is None else _geometry(geometry)
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.tp_row = torch.empty(T * P, **i32)
        self.part_tokens = torch.empty(P, **i32)
        self.part_token_offset = torch.empty(P + 1, **i32)
        self.tp_src = torch.empty(T * P, **i32)
        self.kmask = torch.empty(T * P, **i32)
        self.status = torch.empty(1, **i32)
        self.idx32 = torch.empty((T, K), **i32)          # int64 ids narrowed here
        wsb = ep_dedup_layout_dispatch_workspace_bytes(T, K, E, P)
        self.ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
        if payload == "fp8":
            self.recv_x = torch.empty((T * P, H), dtype=torch.uint8, device=dev)
            self.recv_scales = torch.empty((T * P, H // 128), dtype=torch.float32, device=dev)
        else:
            self.recv_x = torch.empty((T * P, H), dtype=torch.bfloat16, device=dev)
            self.recv_scales = None
        self.partial = torch.empty((T * P, H), dtype=torch.bfloat16, device=dev)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

    def _views(self, n):
        m = n * self.P
        return (self.tp_row[:m], self.tp_src[:m], self.kmask[:m], self.recv_x[:m],
                None if self.recv_scales is None else self.recv_scales[:m], self.partial[:m])

    def layout(self, topk_idx, stream=None):
        """topk_idx int32 [n, K], n <= T, or int64 (narrowed first, one extra
        launch); sets the batch to n tokens."""
        n = _tokens(self, topk_idx)
        topk_idx = _ids32(self, topk_idx, stream)
        tpr, tps, km, _, _, _ = self._views(n)
        ep_dedup_layout(topk_idx, self.E, self.P, tpr, self.part_tokens, self.part_token_offset,
                        tps, km, self.status, self.ws, stream)
        self.n = n

    def layout_dispatch(self, topk_idx, x, plain, stream=None, geometry=None):
        """ep_dedup_layout_dispatch: the per-expert layout into `plain` (an
        EpBuffers of the same shape), the dedup layout and dispatch here.
        geometry: None (the buffers' own, see __init__) or a (waves_per_block,
        max_blocks[, slice_cols]) tuple (ep_dedup_layout_dispatch_geom)."""
        if geometry is None:
            geometry = self.geometry
        n = _tokens(self, topk_idx)
        if n > plain.T:
            raise ValueError("plain buffers hold %d tokens, the batch has %d" % (plain.T, n))
        topk_idx = _ids32(self, topk_idx, stream)
        tpr, tps, km, rx, rs, _ = self._views(n)
        rop, src, _, _ = plain._views(n)
        ep_dedup_layout_dispatch(topk_idx, x, self.E, self.P, self.payload, plain.expert_count,
                                 plain.expert_offset, plain.part_count, plain.part_offset,
                                 rop, src, tpr, self.part_tokens, self.part_token_offset, tps, km,
                                 self.status, self.ws, rx, rs, stream, geometry)
        self.n = plain.n = n

    def plan(self, geometry=None):
        """How layout_dispatch runs this shape (ep_dedup_layout_dispatch_plan),
        with the buffers' own geometry unless one is given."""
        return ep_dedup_layout_dispatch_plan(self.T, self.H, self.K, self.E, self.P, self.payload,
                                             self.geometry if geometry is None else geometry)

    def dispatch(self, x, stream=None):
        """One copy of each token per partition it reaches (ep_dispatch, K = P,
        tp_row); x bf16 [n, H] of the current batch."""
        _same_tokens(self, x.shape[0], "x")
        tpr, _, _, rx, rs, _ = self._views(self.n)
        ep_dispatch(x, self.P, tpr, self.payload, rx, rs, stream)

    def combine_partial(self, expert_out, row_of_pair, topk_w, stream=None):
        """topk_w fp32 [n, K] of the current batch and its row_of_pair (the
        first n*K entries are used, e.g. the plain buffers' whole array);
        returns partial[:n*P]."""
        _same_tokens(self, topk_w.shape[0], "topk_w")
        tpr, _, km, _, _, part = self._views(self.n)
        ep_combine_partial(expert_out, row_of_pair[:self.n * self.K], topk_w, tpr, km, self.P,
                           part, stream)
        return part

    def combine_reduce(self, stream=None):
        """Returns out[:n] of the current batch."""
        tpr, _, _, _, _, part = self._views(self.n)
        out = self.out[:self.n]
        ep_combine_reduce(part, tpr, self.n, self.P, out, stream)
        return out


class BoundStep:
    """ep_layout_dispatch + ep_combine with every argument marshalled once.

    For a serving loop whose buffers never move: the pointers, sizes and stream
    are converted to ctypes values at bind time, so each call is a single
    foreign call with no per-call tensor inspection (the host-side cost that
    paces the GPU at a few tokens; MoRI PR #614, view-cache paragraph).  The
    library still checks every argument on each call.
    """

    def __init__(self, buf, topk_idx, x, expert_out, topk_w, stream=None):
        _dt(topk_idx, torch.int32)
        _dt(x, *_BF16)
        _dt(expert_out, *_BF16)
        _dt(topk_w, torch.float32)
        T, K = topk_idx.shape
        if (T, K) != (buf.T, buf.K) or tuple(x.shape) != (buf.T, buf.H) or \
                tuple(topk_w.shape) != (buf.T, buf.K) or tuple(expert_out.shape) != (buf.T * buf.K, buf.H):
            raise ValueError("tensor shapes do not match the buffers")
        self._keep = (buf, topk_idx, x, expert_out, topk_w, stream)   # keep the memory alive
        s = _stream(stream)
        ws_bytes = buf.ws.numel()
        self._ld = (_ptr(topk_idx), _ptr(x), T, buf.H, K, buf.E, buf.P, PAYLOADS[buf.payload],
                    _ptr(buf.expert_count), _ptr(buf.expert_offset), _ptr(buf.part_count),
                    _ptr(buf.part_offset), _ptr(buf.row_of_pair), _ptr(buf.src_pair),
                    _ptr(buf.status), _ptr(buf.ws), ws_bytes, _ptr(buf.recv_x),
                    _ptr(buf.recv_scales))
        g = buf.geometry.get("layout_dispatch")
        if g is None:
            self._ld = self._ld + (s,)
            self._f_ld = _lib.ep_layout_dispatch
        else:
            self._ld = self._ld + tuple(g) + (s,)
            self._f_ld = _lib.ep_layout_dispatch_geom
        g = buf.geometry.get("combine")
        self._cb = (_ptr(expert_out), _ptr(buf.row_of_pair), _ptr(topk_w), T, buf.H, K,
                    _ptr(buf.out))
        if g is None:
            self._cb = self._cb + (s,)
            self._f_cb = _lib.ep_combine
        else:
            self._cb = self._cb + tuple(g) + (s,)
            self._f_cb = _lib.ep_combine_geom

    def layout_dispatch(self):
        rc = self._f_ld(*self._ld)
        if rc:
            raise EpError("ep_layout_dispatch", rc)

    def combine(self):
        rc = self._f_cb(*self._cb)
        if rc:
            raise EpError("ep_combine", rc)

    def step(self):
        rc = self._f_ld(*self._ld)
        if rc == 0:
            rc = self._f_cb(*self._cb)
        if rc:
            raise EpError("ep_layout_dispatch/ep_combine", rc)
