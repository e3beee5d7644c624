"""CPU checks of the Python binding's argument checks: every wrapper refuses,
before any pointer reaches the library, a tensor whose dtype or size does not
match what the call would read or write on the device (a short buffer would
otherwise be overrun there).  CPU tensors are used: the shape checks come
before the device check, so nothing here touches a GPU."""
import pytest
import torch

import combine_ep_layout_05_amd as ep

T, H, K, E, P = 4, 256, 8, 32, 8
i32 = dict(dtype=torch.int32)


def layout_outputs(**over):
    d = dict(expert_count=torch.empty(E, **i32), expert_offset=torch.empty(E + 1, **i32),
             part_count=torch.empty(P, **i32), part_offset=torch.empty(P + 1, **i32),
             row_of_pair=torch.empty(T * K, **i32), src_pair=torch.empty(T * K, **i32),
             status=torch.empty(1, **i32))
    d.update(over)
    return d


def inputs():
    return dict(idx=torch.zeros(T, K, **i32), x=torch.zeros(T, H, dtype=torch.bfloat16),
                y=torch.zeros(T * K, H, dtype=torch.bfloat16), w=torch.zeros(T, K),
                recv_x=torch.empty(T * K, H, dtype=torch.uint8),
                recv_scales=torch.empty(T * K, H // 128), out=torch.empty(T, H, dtype=torch.bfloat16))


def _layout(**over):
    a = inputs()
    o = layout_outputs(**over)
    ep.ep_layout(a["idx"], E, P, o["expert_count"], o["expert_offset"], o["part_count"],
                 o["part_offset"], o["row_of_pair"], o["src_pair"], o["status"])


@pytest.mark.parametrize("name,bad", [
    ("expert_count", torch.empty(E - 1, **i32)), ("expert_offset", torch.empty(E, **i32)),
    ("part_count", torch.empty(P + 1, **i32)), ("part_offset", torch.empty(P, **i32)),
    ("row_of_pair", torch.empty(T * K - 1, **i32)), ("src_pair", torch.empty(T, **i32)),
])
def test_layout_refuses_short_outputs(name, bad):
    with pytest.raises(ValueError, match=name):
        _layout(**{name: bad})


def test_layout_refuses_wrong_dtypes():
    with pytest.raises(TypeError):
        _layout(row_of_pair=torch.empty(T * K, dtype=torch.int64))
    with pytest.raises(ValueError, match="device tensor"):     # right shapes: the device check
        _layout()


def test_dispatch_checks_payload_buffers():
    a = inputs()
    rop = torch.empty(T * K, **i32)
    # a bf16 payload into a uint8 buffer would write 2x past its end
    with pytest.raises(TypeError):
        ep.ep_dispatch(a["x"], K, rop, "bf16", a["recv_x"])
    # too few receive rows, wrong width, missing or short scales
    with pytest.raises(ValueError, match="recv_x"):
        ep.ep_dispatch(a["x"], K, rop, "fp8", a["recv_x"][:T * K - 1], a["recv_scales"])
    with pytest.raises(ValueError, match="recv_x"):
        ep.ep_dispatch(a["x"], K, rop, "fp8", torch.empty(T * K, H - 128, dtype=torch.uint8),
                       a["recv_scales"])
    with pytest.raises(ValueError, match="recv_scales"):
        ep.ep_dispatch(a["x"], K, rop, "fp8", a["recv_x"], None)
    with pytest.raises(ValueError, match="recv_scales"):
        ep.ep_dispatch(a["x"], K, rop, "fp8", a["recv_x"], a["recv_scales"][:, :1])
    with pytest.raises(ValueError, match="row_of_pair"):
        ep.ep_dispatch(a["x"], K, rop[:-1], "fp8", a["recv_x"], a["recv_scales"])
    # more receive rows than needed is fine (the device check comes next)
    with pytest.raises(ValueError, match="device tensor"):
        ep.ep_dispatch(a["x"], K, rop, "bf16", torch.empty(T * K + 3, H, dtype=torch.bfloat16))


def test_layout_dispatch_checks_everything():
    a = inputs()
    o = layout_outputs()

    def call(x=a["x"], recv_x=a["recv_x"], recv_scales=a["recv_scales"], **kw):
        oo = dict(o, **kw)
        ep.ep_layout_dispatch(a["idx"], x, E, P, "fp8", oo["expert_count"], oo["expert_offset"],
                              oo["part_count"], oo["part_offset"], oo["row_of_pair"],
                              oo["src_pair"], oo["status"], None, recv_x, recv_scales)
    with pytest.raises(ValueError, match="x:"):
        call(x=torch.zeros(T + 1, H, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="part_offset"):
        call(part_offset=torch.empty(P, **i32))
    with pytest.raises(ValueError, match="recv_scales"):
        call(recv_scales=torch.empty(T * K - 1, H // 128))
    with pytest.raises(ValueError, match="device tensor"):
        call()


def test_combine_checks_expert_rows_and_width():
    a = inputs()
    rop = torch.empty(T * K, **i32)
    with pytest.raises(ValueError, match="expert_out"):
        ep.ep_combine(a["y"][:T * K - 1], rop, a["w"], a["out"])
    with pytest.raises(ValueError, match="expert_out"):        # width != out's width
        ep.ep_combine(torch.zeros(T * K, H + 8, dtype=torch.bfloat16), rop, a["w"], a["out"])
    with pytest.raises(ValueError, match="out"):
        ep.ep_combine(a["y"], rop, a["w"], torch.empty(T - 1, H, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="row_of_pair"):
        ep.ep_combine(a["y"], rop[:5], a["w"], a["out"])
    with pytest.raises(TypeError):
        ep.ep_combine(a["y"], rop, a["w"].double(), a["out"])


def test_dedup_wrappers_check_sizes():
    a = inputs()
    tp = torch.empty(T * P, **i32)
    ptok = torch.empty(P, **i32)
    ptoff = torch.empty(P + 1, **i32)
    st = torch.empty(1, **i32)
    with pytest.raises(ValueError, match="kmask"):
        ep.ep_dedup_layout(a["idx"], E, P, tp, ptok, ptoff, tp, tp[:-1], st)
    with pytest.raises(ValueError, match="part_token_offset"):
        ep.ep_dedup_layout(a["idx"], E, P, tp, ptok, ptok, tp, tp, st)
    partial = torch.empty(T * P, H, dtype=torch.bfloat16)
    rop = torch.empty(T * K, **i32)
    with pytest.raises(ValueError, match="partial"):
        ep.ep_combine_partial(a["y"], rop, a["w"], tp, tp, P, partial[:-1])
    with pytest.raises(ValueError, match="tp_row"):
        ep.ep_combine_reduce(partial, tp[:-1], T, P, a["out"])
    with pytest.raises(ValueError, match="partial"):
        ep.ep_combine_reduce(partial[:, :-8], tp, T, P, a["out"])


def test_geometry_tuple_checked():
    with pytest.raises(ValueError, match="geometry"):
        ep.ep_layout_dispatch_plan(128, 7168, 8, 288, 16, "fp8", (1, 2, 3, 4))
