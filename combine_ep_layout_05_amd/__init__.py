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
    "ep_layout_dispatch_noalloc": ([_P, _P, _I, _I, _I, _I, _I, _I] + [_P] * 10, _I),
    "ep_graph_begin": ([_P], _I),
    "ep_graph_end": ([_P, ctypes.POINTER(_P)], _I),
    "ep_graph_launch": ([_P, _P], _I),
    "ep_graph_destroy": ([_P], _I),
    "ep_e4m3fn_encode": ([_P, _I64, _P, _P], _I),
    "ep_dispatch_geom": ([_P, _I, _I, _I, _P, _I, _P, _P, _I, _I, _P], _I),
    "ep_combine_geom": ([_P, _P, _P, _I, _I, _I, _P, _I, _I, _P], _I),
    "ep_dedup_layout_workspace_bytes": ([_I, _I, _I, _I], _SZ),
    "ep_dedup_layout": ([_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], _I),
    "ep_combine_partial": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P], _I),
    "ep_dedup_layout_dispatch_workspace_bytes": ([_I, _I, _I, _I], _SZ),
    "ep_dedup_layout_dispatch": ([_P, _P, _I, _I, _I, _I, _I, _I] + [_P] * 12 + [_P, _SZ, _P, _P, _P],
                                 _I),
    "ep_combine_reduce": ([_P, _P, _I, _I, _I, _P, _P], _I),
    "ep_strerror": ([_I], ctypes.c_char_p),
    "ep_last_hip_error": ([], _I),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes, _f.restype = _args, _res


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


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def library_path() -> str:
    return LIB_PATH


def ep_layout_workspace_bytes(T: int, K: int, E: int) -> int:
    return int(_lib.ep_layout_workspace_bytes(T, K, E))


def ep_layout(topk_idx, E, P, expert_count, expert_offset, part_count, part_offset,
              row_of_pair, src_pair, status, ws=None, stream=None):
    """topk_idx int32 [T, K] -> the layout outputs (see include/ep.h)."""
    _dt(topk_idx, torch.int32)
    for t in (expert_count, expert_offset, part_count, part_offset, row_of_pair, src_pair):
        _dt(t, torch.int32)
    _dt(status, torch.int32, torch.uint32)
    T, K = topk_idx.shape
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("ep_layout", _lib.ep_layout(
        _ptr(topk_idx), T, K, E, P, _ptr(expert_count), _ptr(expert_offset), _ptr(part_count),
        _ptr(part_offset), _ptr(row_of_pair), _ptr(src_pair), _ptr(status), _ptr(ws), ws_bytes,
        _stream(stream)))


def ep_dispatch(x, K, row_of_pair, payload, recv_x, recv_scales=None, stream=None, geometry=None):
    """x bf16 [T, H] -> recv_x (uint8 fp8 bytes or bf16) [T*K, H], recv_scales fp32 [T*K, H/128].
    geometry: None (library default) or (waves_per_block, max_blocks)."""
    _dt(x, torch.bfloat16, torch.int16, torch.uint16)
    _dt(row_of_pair, torch.int32)
    payload = PAYLOADS.get(payload, payload)
    T, H = x.shape
    if geometry is None:
        _check("ep_dispatch", _lib.ep_dispatch(_ptr(x), T, H, K, _ptr(row_of_pair), payload,
                                               _ptr(recv_x), _ptr(recv_scales), _stream(stream)))
    else:
        wv, mb = geometry
        _check("ep_dispatch_geom", _lib.ep_dispatch_geom(
            _ptr(x), T, H, K, _ptr(row_of_pair), payload, _ptr(recv_x), _ptr(recv_scales), wv, mb,
            _stream(stream)))


def ep_layout_dispatch(topk_idx, x, E, P, payload, expert_count, expert_offset, part_count,
                       part_offset, row_of_pair, src_pair, status, ws, recv_x, recv_scales=None,
                       stream=None):
    """ep_layout followed by ep_dispatch, as one launch for small batches."""
    _dt(topk_idx, torch.int32)
    _dt(x, torch.bfloat16, torch.int16, torch.uint16)
    payload = PAYLOADS.get(payload, payload)
    T, K = topk_idx.shape
    H = x.shape[1]
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("ep_layout_dispatch", _lib.ep_layout_dispatch(
        _ptr(topk_idx), _ptr(x), T, H, K, E, P, payload, _ptr(expert_count), _ptr(expert_offset),
        _ptr(part_count), _ptr(part_offset), _ptr(row_of_pair), _ptr(src_pair), _ptr(status),
        _ptr(ws), ws_bytes, _ptr(recv_x), _ptr(recv_scales), _stream(stream)))


def ep_layout_dispatch_noalloc(topk_idx, x, E, P, payload, expert_count, expert_offset,
                               part_count, part_offset, row_of_pair, src_pair, status, recv_x,
                               recv_scales=None, stream=None):
    """ep_layout_dispatch with the library's own per-device scratch buffer as
    the layout workspace: the call allocates nothing (see include/ep.h)."""
    _dt(topk_idx, torch.int32)
    _dt(x, torch.bfloat16, torch.int16, torch.uint16)
    payload = PAYLOADS.get(payload, payload)
    T, K = topk_idx.shape
    H = x.shape[1]
    _check("ep_layout_dispatch_noalloc", _lib.ep_layout_dispatch_noalloc(
        _ptr(topk_idx), _ptr(x), T, H, K, E, P, payload, _ptr(expert_count), _ptr(expert_offset),
        _ptr(part_count), _ptr(part_offset), _ptr(row_of_pair), _ptr(src_pair), _ptr(status),
        _ptr(recv_x), _ptr(recv_scales), _stream(stream)))


def ep_combine(expert_out, row_of_pair, topk_w, out, stream=None, geometry=None):
    """expert_out bf16 [T*K, H] (receive-row layout), topk_w fp32 [T, K] -> out bf16 [T, H].
    geometry: None (library default) or (waves_per_block, max_blocks)."""
    _dt(expert_out, torch.bfloat16, torch.int16, torch.uint16)
    _dt(out, torch.bfloat16, torch.int16, torch.uint16)
    _dt(topk_w, torch.float32)
    _dt(row_of_pair, torch.int32)
    T, K = topk_w.shape
    H = out.shape[1]
    if geometry is None:
        _check("ep_combine", _lib.ep_combine(_ptr(expert_out), _ptr(row_of_pair), _ptr(topk_w), T,
                                             H, K, _ptr(out), _stream(stream)))
    else:
        wv, mb = geometry
        _check("ep_combine_geom", _lib.ep_combine_geom(
            _ptr(expert_out), _ptr(row_of_pair), _ptr(topk_w), T, H, K, _ptr(out), wv, mb,
            _stream(stream)))


def ep_e4m3fn_encode(values_f32, out_u8, stream=None):
    _dt(values_f32, torch.float32)
    _dt(out_u8, torch.uint8)
    _check("ep_e4m3fn_encode", _lib.ep_e4m3fn_encode(_ptr(values_f32), values_f32.numel(),
                                                     _ptr(out_u8), _stream(stream)))


def ep_dedup_layout_workspace_bytes(T: int, K: int, E: int, P: int) -> int:
    return int(_lib.ep_dedup_layout_workspace_bytes(T, K, E, P))


def ep_dedup_layout(topk_idx, E, P, tp_row, part_tokens, part_token_offset, tp_src, kmask,
                    status, ws=None, stream=None):
    """topk_idx int32 [T, K] -> per-destination (dedup) layout (see include/ep.h)."""
    _dt(topk_idx, torch.int32)
    for t in (tp_row, part_tokens, part_token_offset, tp_src):
        _dt(t, torch.int32)
    _dt(kmask, torch.int32, torch.uint32)
    _dt(status, torch.int32, torch.uint32)
    T, K = topk_idx.shape
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("ep_dedup_layout", _lib.ep_dedup_layout(
        _ptr(topk_idx), T, K, E, P, _ptr(tp_row), _ptr(part_tokens), _ptr(part_token_offset),
        _ptr(tp_src), _ptr(kmask), _ptr(status), _ptr(ws), ws_bytes, _stream(stream)))


def ep_dedup_layout_dispatch_workspace_bytes(T: int, K: int, E: int, P: int) -> int:
    return int(_lib.ep_dedup_layout_dispatch_workspace_bytes(T, K, E, P))


def ep_dedup_layout_dispatch(topk_idx, x, E, P, payload, expert_count, expert_offset, part_count,
                             part_offset, row_of_pair, src_pair, tp_row, part_tokens,
                             part_token_offset, tp_src, kmask, status, ws, recv_x,
                             recv_scales=None, stream=None):
    """Per-expert layout + dedup layout + dedup dispatch (one launch for small batches)."""
    _dt(topk_idx, torch.int32)
    _dt(x, torch.bfloat16, torch.int16, torch.uint16)
    payload = PAYLOADS.get(payload, payload)
    T, K = topk_idx.shape
    H = x.shape[1]
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("ep_dedup_layout_dispatch", _lib.ep_dedup_layout_dispatch(
        _ptr(topk_idx), _ptr(x), T, H, K, E, P, payload, _ptr(expert_count), _ptr(expert_offset),
        _ptr(part_count), _ptr(part_offset), _ptr(row_of_pair), _ptr(src_pair), _ptr(tp_row),
        _ptr(part_tokens), _ptr(part_token_offset), _ptr(tp_src), _ptr(kmask), _ptr(status),
        _ptr(ws), ws_bytes, _ptr(recv_x), _ptr(recv_scales), _stream(stream)))


def ep_combine_partial(expert_out, row_of_pair, topk_w, tp_row, kmask, P, partial, stream=None):
    """Level 1: expert_out bf16 [T*K, H] -> partial bf16 [T*P, H] (rows of present couples)."""
    _dt(expert_out, torch.bfloat16, torch.int16, torch.uint16)
    _dt(partial, torch.bfloat16, torch.int16, torch.uint16)
    _dt(topk_w, torch.float32)
    _dt(row_of_pair, torch.int32)
    _dt(tp_row, torch.int32)
    _dt(kmask, torch.int32, torch.uint32)
    T, K = topk_w.shape
    H = partial.shape[1]
    _check("ep_combine_partial", _lib.ep_combine_partial(
        _ptr(expert_out), _ptr(row_of_pair), _ptr(topk_w), _ptr(tp_row), _ptr(kmask), T, H, K, P,
        _ptr(partial), _stream(stream)))


def ep_combine_reduce(partial, tp_row, T, P, out, stream=None):
    """Level 2: partial bf16 [T*P, H] -> out bf16 [T, H] (partition-order fp32 sum)."""
    _dt(partial, torch.bfloat16, torch.int16, torch.uint16)
    _dt(out, torch.bfloat16, torch.int16, torch.uint16)
    _dt(tp_row, torch.int32)
    H = out.shape[1]
    _check("ep_combine_reduce", _lib.ep_combine_reduce(_ptr(partial), _ptr(tp_row), T, H, P,
                                                       _ptr(out), _stream(stream)))


class EpGraph:
    """A recorded sequence of ep_* calls (HIP graph), replayed with ep_graph_launch."""

    def __init__(self, handle):
        self._h = ctypes.c_void_p(handle)

    def launch(self, stream=None):
        _check("ep_graph_launch", _lib.ep_graph_launch(self._h, _stream(stream)))

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
    call, so the calls can be captured into a graph)."""

    def __init__(self, T, H, K, E, P, payload="fp8", device="cuda", geometry=None):
        """geometry: None (library defaults), "tuned" (the saved rules for this
        shape, where there are any) or {"dispatch": (waves, max_blocks),
        "combine": (waves, max_blocks)}."""
        self.T, self.H, self.K, self.E, self.P = T, H, K, E, P
        self.payload = payload
        if geometry == "tuned":
            from . import tuning
            geometry = {ph: tuning.lookup(ph, T, H, K, payload) for ph in ("dispatch", "combine")}
        self.geometry = {k: v for k, v in (geometry or {}).items() if v is not None}
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.expert_count = torch.empty(E, **i32)
        self.expert_offset = torch.empty(E + 1, **i32)
        self.part_count = torch.empty(P, **i32)
        self.part_offset = torch.empty(P + 1, **i32)
        self.row_of_pair = torch.empty(T * K, **i32)
        self.src_pair = torch.empty(T * K, **i32)
        self.status = torch.empty(1, **i32)
        wsb = ep_layout_workspace_bytes(T, K, E)
        self.ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
        if payload == "fp8":
            self.recv_x = torch.empty((T * K, H), dtype=torch.uint8, device=dev)
            self.recv_scales = torch.empty((T * K, H // 128), dtype=torch.float32, device=dev)
        else:
            self.recv_x = torch.empty((T * K, H), dtype=torch.bfloat16, device=dev)
            self.recv_scales = None
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

    def layout(self, topk_idx, stream=None):
        ep_layout(topk_idx, self.E, self.P, self.expert_count, self.expert_offset, self.part_count,
                  self.part_offset, self.row_of_pair, self.src_pair, self.status, self.ws, stream)

    def layout_dispatch(self, topk_idx, x, stream=None):
        ep_layout_dispatch(topk_idx, x, self.E, self.P, self.payload, self.expert_count,
                           self.expert_offset, self.part_count, self.part_offset, self.row_of_pair,
                           self.src_pair, self.status, self.ws, self.recv_x, self.recv_scales, stream)

    def dispatch(self, x, stream=None):
        ep_dispatch(x, self.K, self.row_of_pair, self.payload, self.recv_x, self.recv_scales, stream,
                    self.geometry.get("dispatch"))

    def combine(self, expert_out, topk_w, stream=None):
        ep_combine(expert_out, self.row_of_pair, topk_w, self.out, stream,
                   self.geometry.get("combine"))
        return self.out


class EpDedupBuffers:
    """Persistent device buffers of the per-destination (dedup) path for one
    shape: the dedup layout, the dedup receive rows (one per present (token,
    partition) couple), the partial rows and the output."""

    def __init__(self, T, H, K, E, P, payload="fp8", device="cuda"):
        self.T, self.H, self.K, self.E, self.P = T, H, K, E, P
        self.payload = payload
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.tp_row = torch.empty(T * P, **i32)
        self.part_tokens = torch.empty(P, **i32)
        self.part_token_offset = torch.empty(P + 1, **i32)
        self.tp_src = torch.empty(T * P, **i32)
        self.kmask = torch.empty(T * P, **i32)
        self.status = torch.empty(1, **i32)
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

    def layout(self, topk_idx, stream=None):
        ep_dedup_layout(topk_idx, self.E, self.P, self.tp_row, self.part_tokens,
                        self.part_token_offset, self.tp_src, self.kmask, self.status, self.ws,
                        stream)

    def layout_dispatch(self, topk_idx, x, plain, stream=None):
        """ep_dedup_layout_dispatch: the per-expert layout into `plain` (an
        EpBuffers of the same shape), the dedup layout and dispatch here."""
        ep_dedup_layout_dispatch(topk_idx, x, self.E, self.P, self.payload, plain.expert_count,
                                 plain.expert_offset, plain.part_count, plain.part_offset,
                                 plain.row_of_pair, plain.src_pair, self.tp_row, self.part_tokens,
                                 self.part_token_offset, self.tp_src, self.kmask, self.status,
                                 self.ws, self.recv_x, self.recv_scales, stream)

    def dispatch(self, x, stream=None):
        """One copy of each token per partition it reaches (ep_dispatch, K = P, tp_row)."""
        ep_dispatch(x, self.P, self.tp_row, self.payload, self.recv_x, self.recv_scales, stream)

    def combine_partial(self, expert_out, row_of_pair, topk_w, stream=None):
        ep_combine_partial(expert_out, row_of_pair, topk_w, self.tp_row, self.kmask, self.P,
                           self.partial, stream)
        return self.partial

    def combine_reduce(self, stream=None):
        ep_combine_reduce(self.partial, self.tp_row, self.T, self.P, self.out, stream)
        return self.out


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
        _dt(x, torch.bfloat16, torch.int16, torch.uint16)
        _dt(expert_out, torch.bfloat16, torch.int16, torch.uint16)
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
                    _ptr(buf.recv_scales), s)
        g = buf.geometry.get("combine")
        if g is None:
            self._cb = (_ptr(expert_out), _ptr(buf.row_of_pair), _ptr(topk_w), T, buf.H, K,
                        _ptr(buf.out), s)
            self._f_cb = _lib.ep_combine
        else:
            self._cb = (_ptr(expert_out), _ptr(buf.row_of_pair), _ptr(topk_w), T, buf.H, K,
                        _ptr(buf.out), int(g[0]), int(g[1]), s)
            self._f_cb = _lib.ep_combine_geom
        self._f_ld = _lib.ep_layout_dispatch

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
