"""int8 weight x int8 activation GEMV on the GPU: the int32 accumulators must
equal the oracle's bit for bit, the rescaled fp32 output must be within the
floating-point bound."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_bits_equal, assert_within, dev, host, say
from weight_streaming_gemv_decode_amd import synth, wsgemv

pytestmark = pytest.mark.gpu


def _case(N, K, workload=4, ids=(0, 1, 2)):
    Wq = synth.int8_uniform(workload, ids[0], (N, K))
    xq = synth.int8_uniform(workload, ids[1], (K,))
    s_w = synth.f32_uniform(workload, ids[2], (N,), 0.001, 0.01)
    return Wq, xq, s_w


def _run(Wq, xq, s_w, s_x=synth.X_SCALE_W8A8, splits=0):
    xs = torch.tensor([s_x], dtype=torch.float32, device="cuda")
    y, acc = wsgemv.gemv_w8a8(dev(Wq), dev(s_w), dev(xq), xs, splits=splits)
    return host(y), host(acc)


def _check(Wq, xq, s_w, y, acc, what, s_x=synth.X_SCALE_W8A8):
    acc_ref, y_ref, A = oracle.gemv_w8a8(Wq, s_w, xq, s_x)
    assert_bits_equal(acc, acc_ref, f"{what} int32 accumulators")
    assert_within(y, y_ref, A, what)


@pytest.mark.parametrize("N,K", synth.C4_SHAPES)
def test_c4_shapes(N, K):
    say(f"w8a8 {N}x{K} auto")
    Wq, xq, s_w = _case(N, K, ids=(10 * (K // 4096), 1 + 10 * (K // 4096), 2 + 10 * (K // 4096)))
    y, acc = _run(Wq, xq, s_w)
    _check(Wq, xq, s_w, y, acc, f"{N}x{K}")


@pytest.mark.parametrize("S", [1, 2, 7, 14])
def test_c4b_splits(S):
    N, K = 4096, 14336
    say(f"w8a8 {N}x{K} S={S}")
    Wq, xq, s_w = _case(N, K)
    y, acc = _run(Wq, xq, s_w, splits=S)
    _check(Wq, xq, s_w, y, acc, f"S={S}")
    y2, acc2 = _run(Wq, xq, s_w, splits=S)
    assert_bits_equal(y2, y, "repeat y")


@pytest.mark.parametrize("N,K", [(1, 16), (3, 48), (17, 1008), (65, 2064), (129, 4112), (2, 32768), (5, 33024)])
def test_ragged_shapes(N, K):
    say(f"w8a8 ragged {N}x{K}")
    Wq, xq, s_w = _case(N, K, workload=60, ids=(N, K, N + K))
    y, acc = _run(Wq, xq, s_w)
    _check(Wq, xq, s_w, y, acc, f"{N}x{K}")


def test_minus_128_and_int32_extremes():
    say("w8a8 extremes")
    K = 16384
    Wq = np.full((4, K), 127, np.int8)
    Wq[1] = -128
    Wq[2, ::2] = -128
    Wq[3] = np.where(np.arange(K) % 3 == 0, -128, 127).astype(np.int8)
    xq = np.full(K, 127, np.int8)
    xq[1::4] = -128
    s_w = np.array([1.0, 0.5, 0.25, 2.0], np.float32)
    y, acc = _run(Wq, xq, s_w, s_x=1.0)
    _check(Wq, xq, s_w, y, acc, "extremes", s_x=1.0)


def test_acc_out_optional_and_degenerate():
    say("w8a8 no acc_out, K=0")
    Wq, xq, s_w = _case(64, 256, workload=61)
    xs = torch.tensor([0.02], dtype=torch.float32, device="cuda")
    y, acc = wsgemv.gemv_w8a8(dev(Wq), dev(s_w), dev(xq), xs, want_acc=False)
    assert acc is None
    _, y_ref, A = oracle.gemv_w8a8(Wq, s_w, xq, 0.02)
    assert_within(host(y), y_ref, A, "no acc_out")
    y = torch.full((3,), 5.0, device="cuda")
    acc = torch.full((3,), 9, dtype=torch.int32, device="cuda")
    wsgemv.gemv_w8a8(torch.empty((3, 0), dtype=torch.int8, device="cuda"), torch.ones(3, device="cuda"),
                     torch.empty(0, dtype=torch.int8, device="cuda"), xs, y=y, acc_out=acc)
    assert host(y).tolist() == [0.0] * 3 and host(acc).tolist() == [0] * 3
