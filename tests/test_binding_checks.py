"""The Python binding's checks of a decode-step linear, on the CPU.

wsgemv.Linear checks every tensor against the sizes given beside it (dtype,
contiguity, element count or packed byte count) before it checks where the
tensors live, and all of it before a plan is created: a mis-sized buffer in a
plan would otherwise become an out-of-bounds access inside a kernel.  CPU
tensors are used, so a correctly sized linear stops at the device check,
and a mis-sized one at the size check.
"""
import pytest
import torch

from weight_streaming_gemv_decode_amd import wsgemv

f16, f32, i8, i32, u8 = torch.float16, torch.float32, torch.int8, torch.int32, torch.uint8


def z(*shape, dtype=f32):
    return torch.zeros(shape, dtype=dtype)


def make(kind, **over):
    """A correctly sized CPU linear of each kind, with `over` replacing fields."""
    N, K, M = 40, 256, 1
    if kind == wsgemv.F16:
        a = dict(W=z(N, K, dtype=f16), x=z(K, dtype=f16))
    elif kind == wsgemv.W8A8:
        a = dict(W=z(N, K, dtype=i8), x=z(K, dtype=i8), scale=z(N), x_scale=z(1), acc_out=z(N, dtype=i32))
    elif kind == wsgemv.W8A8_DYN:
        a = dict(W=z(N, K, dtype=i8), x=z(K, dtype=f16), scale=z(N), acc_out=z(N, dtype=i32))
    else:
        M = over.pop("M", 1)
        wb, sb = wsgemv.packed_w4_bytes(N, K)
        a = dict(W=z(wb, dtype=u8), x=z(M, K, dtype=f16), scale=z(sb, dtype=u8), group=128, M=M)
    a.update(dict(y=z(M * N), N=N, K=K))
    a.update(over)
    W, x, y = a.pop("W"), a.pop("x"), a.pop("y")
    return lambda: wsgemv.Linear(kind, W, x, y, a.pop("N"), a.pop("K"), **a)


@pytest.mark.parametrize("kind", [wsgemv.F16, wsgemv.W8A8, wsgemv.W8A8_DYN, wsgemv.W4A16, wsgemv.W4A8])
def test_sized_right_stops_at_the_device(kind):
    with pytest.raises(ValueError, match="must be on a GPU device"):
        make(kind)()


@pytest.mark.parametrize("kind,field,bad,msg", [
    (wsgemv.F16, "y", z(39), "y must hold 40"),
    (wsgemv.F16, "x", z(255, dtype=f16), "x must hold 256"),
    (wsgemv.F16, "W", z(40, 248, dtype=f16), "W must hold"),
    (wsgemv.F16, "W", z(40, 256), "W must be one of"),
    (wsgemv.F16, "x", z(512, dtype=f16)[::2], "x must be contiguous"),
    (wsgemv.W8A8, "scale", z(39), "scale must hold 40"),
    (wsgemv.W8A8, "x_scale", z(2), "x_scale must hold 1"),
    (wsgemv.W8A8, "acc_out", z(40), "acc_out must be one of"),
    (wsgemv.W8A8, "x", z(256, dtype=f16), "x must be one of"),
    (wsgemv.W8A8_DYN, "x", z(256, dtype=i8), "x must be one of"),
    (wsgemv.W4A16, "W", z(100, dtype=u8), "W \\(packed\\) must hold at least"),
    (wsgemv.W4A16, "scale", z(16, dtype=u8), "scale \\(packed\\) must hold at least"),
    (wsgemv.W4A8, "x", z(1, 128, dtype=f16), "x must hold 256"),
    (wsgemv.F16, "argmax_idx", z(2, dtype=i32), "argmax_idx must hold 1"),
    (wsgemv.F16, "argmax_val", z(1, dtype=f16), "argmax_val must be one of"),
    (wsgemv.F16, "y16", z(39, dtype=f16), "y16 must hold at least 80 bytes"),
])
def test_mis_sized_tensor_raises_before_the_plan(kind, field, bad, msg):
    with pytest.raises((ValueError, TypeError), match=msg):
        make(kind, **{field: bad})()


def test_verify_block_x_rows():
    # M = 4 verify block: x must hold M * K values and y M * N
    with pytest.raises(ValueError, match="x must hold 1024"):
        make(wsgemv.W4A16, M=4, x=z(2, 256, dtype=f16))()
    with pytest.raises(ValueError, match="y must hold 160"):
        make(wsgemv.W4A16, M=4, y=z(40))()


def test_conv_tensors():
    N, W = 40, 4
    good = dict(conv_w=z(N, W, dtype=f16), conv_bias=z(N), conv_state=z(N, W - 1), conv_out=z(N))
    with pytest.raises(ValueError, match="must be on a GPU device"):
        make(wsgemv.F16, **good)()
    for field, bad, msg in [("conv_state", z(N, W), "conv_state must hold 120"), ("conv_out", z(N - 1), "conv_out"),
                            ("conv_bias", z(N + 1), "conv_bias"), ("conv_w", z(N, W), "conv_w must be one of")]:
        with pytest.raises((ValueError, TypeError), match=msg):
            make(wsgemv.F16, **{**good, field: bad})()
