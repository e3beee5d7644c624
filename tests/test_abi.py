"""CPU checks of the C ABI: the library loads, exports every symbol the header
declares, and rejects bad arguments on the host before touching the GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ep.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(ep_[a-z0-9_]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    import torch  # noqa: F401  (the HIP runtime is loaded through torch first)
    import combine_ep_layout_05_amd as ep
    return ctypes.CDLL(ep.library_path())


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("ep_layout", "ep_dispatch", "ep_combine", "ep_layout_workspace_bytes",
              "ep_strerror", "ep_last_hip_error", "ep_graph_begin", "ep_graph_end",
              "ep_graph_launch", "ep_graph_destroy", "ep_e4m3fn_encode", "ep_layout_dispatch",
              "ep_dedup_layout", "ep_dedup_layout_workspace_bytes", "ep_combine_partial",
              "ep_combine_reduce", "ep_dedup_layout_dispatch",
              "ep_dedup_layout_dispatch_workspace_bytes", "ep_dispatch_geom", "ep_combine_geom",
              "ep_layout_dispatch_geom", "ep_layout_dispatch_plan", "ep_layout_dispatch_noalloc",
              "ep_dedup_layout_dispatch_geom", "ep_dedup_layout_dispatch_plan",
              "ep_combine_plan", "ep_topk_idx_narrow"):
        assert n in names, n


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_host_side_validation(lib):
    P = ctypes.c_void_p
    L = lib
    L.ep_layout.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int] + [P] * 7 + [
        P, ctypes.c_size_t, P]
    L.ep_dispatch.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, ctypes.c_int, P, P, P]
    L.ep_combine.argtypes = [P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P]
    L.ep_layout_workspace_bytes.restype = ctypes.c_size_t
    L.ep_strerror.restype = ctypes.c_char_p
    fake = P(0x10000)          # never dereferenced: every case below fails a host check first
    odd = P(0x10004)
    ws = [fake] * 7
    # E % P != 0, K out of range, E too large, T < 0
    assert L.ep_layout(fake, 4, 8, 30, 8, *ws, None, 0, None) == -1
    assert L.ep_layout(fake, 4, 17, 32, 8, *ws, None, 0, None) == -1
    assert L.ep_layout(fake, 4, 8, 2048, 8, *ws, None, 0, None) == -1
    assert L.ep_layout(fake, -1, 8, 32, 8, *ws, None, 0, None) == -1
    # null outputs, and a large batch without its workspace
    assert L.ep_layout(fake, 4, 8, 32, 8, None, *ws[1:], None, 0, None) == -1
    assert L.ep_layout_workspace_bytes(4096, 8, 256) > 0
    assert L.ep_layout(fake, 4096, 8, 256, 8, *ws, None, 0, None) == -1
    # dispatch: bad payload, H not a multiple of 128 for fp8, misaligned x
    assert L.ep_dispatch(fake, 4, 1024, 8, fake, 7, fake, fake, None) == -2
    assert L.ep_dispatch(fake, 4, 1000, 8, fake, 0, fake, fake, None) == -1
    assert L.ep_dispatch(odd, 4, 1024, 8, fake, 0, fake, fake, None) == -1
    # combine: H % 8 != 0, null out
    assert L.ep_combine(fake, fake, fake, 4, 1001, 8, fake, None) == -1
    assert L.ep_combine(fake, fake, fake, 4, 1024, 8, None, None) == -1
    # empty batches are accepted without launching anything
    assert L.ep_dispatch(None, 0, 1024, 8, None, 0, None, None, None) == 0
    assert L.ep_combine(None, None, None, 0, 1024, 8, None, None) == 0
    assert b"invalid" in L.ep_strerror(-1)


def test_dedup_host_side_validation(lib):
    P, I = ctypes.c_void_p, ctypes.c_int
    L = lib
    L.ep_dedup_layout.argtypes = [P, I, I, I, I] + [P] * 6 + [P, ctypes.c_size_t, P]
    L.ep_dedup_layout_workspace_bytes.argtypes = [I, I, I, I]
    L.ep_dedup_layout_workspace_bytes.restype = ctypes.c_size_t
    L.ep_combine_partial.argtypes = [P] * 5 + [I, I, I, I, P, P]
    L.ep_combine_reduce.argtypes = [P, P, I, I, I, P, P]
    fake = P(0x10000)          # never dereferenced: every case below fails a host check first
    odd = P(0x10004)
    outs = [fake] * 6
    # P above 16, E % P != 0, P = 0
    assert L.ep_dedup_layout(fake, 4, 8, 64, 32, *outs, None, 0, None) == -1
    assert L.ep_dedup_layout(fake, 4, 8, 30, 8, *outs, None, 0, None) == -1
    assert L.ep_dedup_layout(fake, 4, 8, 32, 0, *outs, None, 0, None) == -1
    # null kmask; a chunked batch without its workspace
    assert L.ep_dedup_layout(fake, 4, 8, 32, 8, *outs[:4], None, fake, None, 0, None) == -1
    assert L.ep_dedup_layout_workspace_bytes(4096, 8, 256, 8) > 0
    assert L.ep_dedup_layout_workspace_bytes(4, 8, 256, 32) == 0
    assert L.ep_dedup_layout(fake, 4096, 8, 256, 8, *outs, None, 0, None) == -1
    # combine levels: P out of range, H % 8, misaligned partial
    assert L.ep_combine_partial(fake, fake, fake, fake, fake, 4, 1024, 8, 17, fake, None) == -1
    assert L.ep_combine_partial(fake, fake, fake, fake, fake, 4, 1001, 8, 8, fake, None) == -1
    assert L.ep_combine_partial(fake, fake, fake, fake, fake, 4, 1024, 8, 8, odd, None) == -1
    assert L.ep_combine_reduce(fake, fake, 4, 1024, 0, fake, None) == -1
    assert L.ep_combine_reduce(odd, fake, 4, 1024, 8, fake, None) == -1
    # empty batches launch nothing
    assert L.ep_combine_partial(None, None, None, None, None, 0, 1024, 8, 8, None, None) == 0
    assert L.ep_combine_reduce(None, None, 0, 1024, 8, None, None) == 0


def test_dedup_layout_dispatch_host_side_validation(lib):
    P, I = ctypes.c_void_p, ctypes.c_int
    L = lib
    L.ep_dedup_layout_dispatch.argtypes = [P, P, I, I, I, I, I, I] + [P] * 12 + [P, ctypes.c_size_t,
                                                                               P, P, P]
    L.ep_dedup_layout_dispatch_workspace_bytes.argtypes = [I, I, I, I]
    L.ep_dedup_layout_dispatch_workspace_bytes.restype = ctypes.c_size_t
    fake = P(0x10000)
    outs = [fake] * 12
    # bad payload; P above 16; fp8 with H % 128 != 0; misaligned x
    assert L.ep_dedup_layout_dispatch(fake, fake, 4, 1024, 8, 32, 8, 5, *outs, None, 0, fake, fake,
                                      None) == -2
    assert L.ep_dedup_layout_dispatch(fake, fake, 4, 1024, 8, 64, 32, 0, *outs, None, 0, fake, fake,
                                      None) == -1
    assert L.ep_dedup_layout_dispatch(fake, fake, 4, 1000, 8, 32, 8, 0, *outs, None, 0, fake, fake,
                                      None) == -1
    assert L.ep_dedup_layout_dispatch(fake, P(0x10004), 4, 1024, 8, 32, 8, 0, *outs, None, 0, fake,
                                      fake, None) == -1
    # a large batch needs the larger of the two layouts' workspaces
    need = L.ep_dedup_layout_dispatch_workspace_bytes(4096, 8, 256, 8)
    assert need >= L.ep_layout_workspace_bytes(4096, 8, 256) > 0
    assert L.ep_dedup_layout_dispatch(fake, fake, 4096, 1024, 8, 256, 8, 0, *outs, fake, need - 16,
                                      fake, fake, None) == -1


def test_geometry_host_side_validation(lib):
    P, I = ctypes.c_void_p, ctypes.c_int
    L = lib
    L.ep_dispatch_geom.argtypes = [P, I, I, I, P, I, P, P, I, I, I, P]
    L.ep_combine_geom.argtypes = [P, P, P, I, I, I, P, I, I, I, P]
    fake = P(0x10000)
    for wv, mb, sc in [(3, 0, 0), (0, 0, 0), (16, 0, 0), (4, -1, 0), (4, 0, 256), (4, 0, 2048)]:
        assert L.ep_dispatch_geom(fake, 4, 1024, 8, fake, 0, fake, fake, wv, mb, sc, None) == -1
        assert L.ep_combine_geom(fake, fake, fake, 4, 1024, 8, fake, wv, mb, sc, None) == -1
    # valid geometry, empty batch: accepted, nothing launched
    assert L.ep_dispatch_geom(None, 0, 1024, 8, None, 0, None, None, 8, 0, 1024, None) == 0
    assert L.ep_combine_geom(None, None, None, 0, 1024, 8, None, 1, 256, 512, None) == 0


def test_layout_dispatch_geom_host_side_validation(lib):
    """A fused batch takes only a workgroup size its kernel accepts; the plan
    query agrees with what the call accepts (host only, nothing launched)."""
    P, I = ctypes.c_void_p, ctypes.c_int
    L = lib
    L.ep_layout_dispatch_geom.argtypes = [P, P, I, I, I, I, I, I] + [P] * 7 + [P, ctypes.c_size_t,
                                                                              P, P, I, I, I, P]
    L.ep_layout_dispatch_plan.argtypes = [I] * 9 + [P]
    fake = P(0x10000)
    outs = [fake] * 7
    plan = (ctypes.c_int32 * 4)()
    pp = ctypes.cast(plan, P)
    for geom in [(4, 256, 0), (4, 0, 1024), (3, 0, 0), (16, 0, 0), (-1, 0, 0)]:
        # 128 x 7168 top-8 runs fused: no cap, no 1024-column slice, 4/6/7/8 waves only
        assert L.ep_layout_dispatch_plan(128, 7168, 8, 288, 16, 0, *geom, pp) == -1
        assert L.ep_layout_dispatch_geom(fake, fake, 128, 7168, 8, 288, 16, 0, *outs, None, 0,
                                         fake, fake, *geom, None) == -1
    assert L.ep_layout_dispatch_plan(128, 7168, 8, 288, 16, 0, 0, 0, 0, pp) == 0
    assert list(plan) == [1, 7, 257, 512]
    assert L.ep_layout_dispatch_plan(4, 6144, 8, 256, 16, 0, 8, 0, 0, pp) == 0
    assert list(plan) == [0, 8, 4 * 12 // 8 + 1, 512]
    assert L.ep_layout_dispatch_plan(4096, 7168, 8, 256, 8, 0, 2, 256, 1024, pp) == 0
    assert list(plan) == [3, 2, 256, 1024]
    assert L.ep_layout_dispatch_plan(4, 6144, 8, 256, 16, 7, 0, 0, 0, pp) == -2
    assert L.ep_layout_dispatch_plan(4, 6144, 8, 256, 16, 0, 0, 0, 0, None) == -1


def test_topk_idx_narrow_host_validation(lib):
    """Rejections happen on the host, before anything is enqueued (fake
    pointers are never dereferenced: every call here returns before a
    launch); n = 0 is a no-op whatever the pointers."""
    P = ctypes.c_void_p
    L = lib
    L.ep_topk_idx_narrow.argtypes = [P, ctypes.c_int64, P, P]
    fake = 0x10000
    assert L.ep_topk_idx_narrow(P(fake), -1, P(fake), None) == -1
    assert L.ep_topk_idx_narrow(None, 0, None, None) == 0
    assert L.ep_topk_idx_narrow(None, 4, P(fake), None) == -1
    assert L.ep_topk_idx_narrow(P(fake), 4, None, None) == -1
    assert L.ep_topk_idx_narrow(P(fake + 4), 4, P(fake), None) == -1     # int64 input 8-B aligned
    assert L.ep_topk_idx_narrow(P(fake), 4, P(fake + 2), None) == -1     # int32 output 4-B aligned


def test_combine_plan(lib):
    """ep_combine's own geometry: 4 waves per workgroup while the combine's
    gathered rows stay below 64 MiB (cached), 2 waves once they stream; a
    given geometry is reported as ep_combine_geom would launch it, one it
    would reject is rejected (host only, nothing launched)."""
    P, I = ctypes.c_void_p, ctypes.c_int
    L = lib
    L.ep_combine_plan.argtypes = [I] * 6 + [P]
    plan = (ctypes.c_int32 * 4)()
    pp = ctypes.cast(plan, P)
    assert L.ep_combine_plan(128, 7168, 8, 0, 0, 0, pp) == 0
    assert list(plan) == [4, 0, 512, 0]
    assert L.ep_combine_plan(4096, 7168, 8, 0, 0, 0, pp) == 0
    assert list(plan) == [2, 0, 512, 1]
    assert L.ep_combine_plan(16384, 4096, 8, 0, 0, 0, pp) == 0
    assert list(plan) == [2, 0, 512, 1]
    # the threshold: T*K*H*2 bytes of gathered rows reaching 64 MiB
    assert L.ep_combine_plan(4096, 1024, 8, 0, 0, 0, pp) == 0 and plan[3] == 1 and plan[0] == 2
    assert L.ep_combine_plan(4095, 1024, 8, 0, 0, 0, pp) == 0 and plan[3] == 0 and plan[0] == 4
    assert L.ep_combine_plan(4096, 7168, 8, 8, 256, 1024, pp) == 0
    assert list(plan) == [8, 256, 1024, 1]
    assert L.ep_combine_plan(0, 7168, 8, 0, 0, 0, pp) == 0
    assert list(plan) == [4, 0, 512, 0]
    plan[0] = 99
    for args in [(4, 7168, 8, 3, 0, 0), (4, 7168, 8, 0, 256, 0), (4, 7168, 8, 0, 0, 1024),
                 (4, 7168, 8, 4, 0, 768), (4, 7168, 8, 4, -1, 0), (4, 7168, 0, 0, 0, 0),
                 (4, 7168, 17, 0, 0, 0), (4, 7164, 8, 0, 0, 0), (-1, 7168, 8, 0, 0, 0)]:
        assert L.ep_combine_plan(*args, pp) == -1, args
    assert plan[0] == 99                                  # untouched on error
    assert L.ep_combine_plan(4, 7168, 8, 0, 0, 0, None) == -1


def test_dedup_layout_dispatch_geom_host_side_validation(lib):
    """ep_dedup_layout_dispatch_geom / _plan: the counting kernel takes 6, 7 or
    8 waves that divide the 512-column steps per token, the general kernel 4
    or 8, a fused batch no cap and no 1024-column slice; a large batch takes
    the dispatch geometry.  Rejections happen on the host (fake pointers are
    never dereferenced)."""
    P, I = ctypes.c_void_p, ctypes.c_int
    L = lib
    L.ep_dedup_layout_dispatch_geom.argtypes = ([P, P, I, I, I, I, I, I] + [P] * 12
                                                + [P, ctypes.c_size_t, P, P, I, I, I, P])
    L.ep_dedup_layout_dispatch_plan.argtypes = [I] * 9 + [P]
    fake = P(0x10000)
    outs = [fake] * 12
    plan = (ctypes.c_int32 * 4)()
    pp = ctypes.cast(plan, P)
    # 128 x 7168 top-8 (14 steps per token): the counting kernel with 7 waves by default
    assert L.ep_dedup_layout_dispatch_plan(128, 7168, 8, 288, 16, 0, 0, 0, 0, pp) == 0
    assert list(plan) == [1, 7, 128 * 14 // 7 + 1, 512]
    # 8 waves do not divide 14 steps: the general kernel; 4 waves too
    assert L.ep_dedup_layout_dispatch_plan(128, 7168, 8, 288, 16, 0, 8, 0, 0, pp) == 0
    assert list(plan) == [2, 8, 128 * 14 // 8, 512]
    assert L.ep_dedup_layout_dispatch_plan(128, 7168, 8, 288, 16, 0, 4, 0, 0, pp) == 0
    assert list(plan) == [2, 4, 128 * 14 // 4, 512]
    # 24 steps per token (hidden 12288): 8 by default, 6 on request; 7 is no size it takes
    assert L.ep_dedup_layout_dispatch_plan(64, 12288, 8, 256, 8, 0, 0, 0, 0, pp) == 0
    assert list(plan) == [1, 8, 64 * 24 // 8 + 1, 512]
    assert L.ep_dedup_layout_dispatch_plan(64, 12288, 8, 256, 8, 0, 6, 0, 0, pp) == 0
    assert list(plan) == [1, 6, 64 * 24 // 6 + 1, 512]
    for geom in [(7, 0, 0), (6, 0, 0), (2, 0, 0)]:
        bad = 12288 if geom[0] == 7 else 7168
        assert L.ep_dedup_layout_dispatch_plan(64, bad, 8, 256, 8, 0, *geom, pp) == -1
        assert L.ep_dedup_layout_dispatch_geom(fake, fake, 64, bad, 8, 256, 8, 0, *outs, None, 0,
                                               fake, fake, *geom, None) == -1
    # a fused batch takes no cap and no 1024-column slice
    for geom in [(4, 256, 0), (4, 0, 1024)]:
        assert L.ep_dedup_layout_dispatch_plan(128, 7168, 8, 288, 16, 0, *geom, pp) == -1
        assert L.ep_dedup_layout_dispatch_geom(fake, fake, 128, 7168, 8, 288, 16, 0, *outs, None,
                                               0, fake, fake, *geom, None) == -1
    # 640 tokens (5120 entries): the layouts, then the dispatch with its geometry
    assert L.ep_dedup_layout_dispatch_plan(640, 7168, 8, 256, 8, 0, 2, 256, 1024, pp) == 0
    assert list(plan) == [3, 2, 256, 1024]
    assert L.ep_dedup_layout_dispatch_plan(640, 7168, 8, 256, 8, 0, 0, 0, 0, pp) == 0
    assert list(plan) == [3, 4, 0, 512]
    for geom in [(3, 0, 0), (4, -1, 0), (4, 0, 768)]:
        assert L.ep_dedup_layout_dispatch_plan(640, 7168, 8, 256, 8, 0, *geom, pp) == -1
    # other arguments: checked as ep_dedup_layout_dispatch checks them
    assert L.ep_dedup_layout_dispatch_plan(4, 1024, 8, 64, 32, 0, 0, 0, 0, pp) == -1
    assert L.ep_dedup_layout_dispatch_plan(4, 1024, 8, 32, 8, 5, 0, 0, 0, pp) == -2
    assert L.ep_dedup_layout_dispatch_plan(4, 1024, 8, 32, 8, 0, 0, 0, 0, None) == -1
    assert L.ep_dedup_layout_dispatch_geom(fake, P(0x10004), 4, 1024, 8, 32, 8, 0, *outs, None, 0,
                                           fake, fake, 0, 0, 0, None) == -1


def test_noalloc_host_side_validation(lib):
    """ep_layout_dispatch_noalloc refuses, before any HIP call, a batch whose
    layout workspace exceeds EP_NOALLOC_SCRATCH_BYTES (EP_ESCRATCH), and
    otherwise checks its arguments as ep_layout_dispatch does."""
    P, I = ctypes.c_void_p, ctypes.c_int
    L = lib
    L.ep_layout_dispatch_noalloc.argtypes = [P, P, I, I, I, I, I, I] + [P] * 10
    L.ep_layout_workspace_bytes.argtypes = [I, I, I]
    L.ep_layout_workspace_bytes.restype = ctypes.c_size_t
    L.ep_strerror.restype = ctypes.c_char_p
    fake = P(0x10000)          # never dereferenced: every case below fails a host check first
    outs = [fake] * 7
    assert L.ep_layout_workspace_bytes(73728, 16, 1024) > (4 << 20)
    assert L.ep_layout_dispatch_noalloc(fake, fake, 73728, 128, 16, 1024, 8, 0, *outs, fake, fake,
                                        None) == -4
    assert b"scratch" in L.ep_strerror(-4)
    # the ordinary argument errors come first
    assert L.ep_layout_dispatch_noalloc(fake, fake, 4, 1024, 8, 32, 8, 5, *outs, fake, fake,
                                        None) == -2
    assert L.ep_layout_dispatch_noalloc(fake, fake, 4, 1000, 8, 32, 8, 0, *outs, fake, fake,
                                        None) == -1
    assert L.ep_layout_dispatch_noalloc(fake, fake, 4, 1024, 8, 30, 8, 0, *outs, fake, fake,
                                        None) == -1
