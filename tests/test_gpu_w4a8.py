"""INT4 weights x INT8 activations (W4A8) on the GPU: the per-token int8
codes and scale the kernel derives from fp16 x, bit for bit against the
oracle's quantiser, and the product within the parity bound against the
oracle's W4A8 product on the oracle's own codes."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_bits_equal, assert_within, dev, host, say
from weight_streaming_gemv_decode_amd import synth, wsgemv

pytestmark = pytest.mark.gpu


def _case(N, K, workload=90, ids=(0, 1, 2), x_sigma=synth.X_SIGMA):
    Wc = synth.w4_words(workload, ids[0], N, K)
    s4 = synth.f16_uniform(workload, ids[1], (N, K // 128), 0.002, 0.02)
    x = synth.f16_normal(workload, ids[2], (K,), x_sigma)
    return Wc, s4, x


def _run(Wc, s4, x, splits=0):
    N, K = Wc.shape[0], x.shape[0]
    Wp, Sp = wsgemv.pack_w4(dev(Wc), dev(s4))
    xq = torch.full((K,), 99, dtype=torch.int8, device="cuda")
    sx = torch.full((1,), float("nan"), device="cuda")
    y = wsgemv.gemv_w4a8(Wp, Sp, dev(x), N, xq_out=xq, sx_out=sx, splits=splits)
    return host(y), host(xq), host(sx)


def _check(Wc, s4, x, splits=0, what=""):
    y, xq, sx = _run(Wc, s4, x, splits)
    xq_ref, sx_ref = oracle.quantize_x_i8(x)
    assert_bits_equal(xq, xq_ref, f"{what} codes")
    assert_bits_equal(sx, np.array([sx_ref], np.float32), f"{what} scale")
    y_ref, A = oracle.gemv_w4a8(Wc, s4, xq_ref, sx_ref)
    assert_within(y, y_ref, A, what)


@pytest.mark.parametrize("N,K", [(1, 128), (16, 128), (17, 256), (100, 640), (2048, 1024), (1024, 3072),
                                 (33, 4096), (5, 8192), (300, 14336)])
def test_shapes(N, K):
    say(f"w4a8 {N}x{K}")
    Wc, s4, x = _case(N, K, ids=(N, K, N + K))
    _check(Wc, s4, x, what=f"{N}x{K}")


@pytest.mark.parametrize("S", [1, 2, 3, 6])
def test_splits(S):
    say(f"w4a8 1024x3072 S={S}")
    Wc, s4, x = _case(1024, 3072, workload=91)
    _check(Wc, s4, x, splits=S, what=f"S={S}")


def test_exact_integer_case():
    """Unit scales and integer activations whose largest magnitude is 127:
    s_x = 1 and xq = x exactly, every partial sum is an integer below 2^24,
    so the fp32 result equals the exact integer product."""
    say("w4a8 exact integers")
    N, K = 300, 1024
    Wc = synth.w4_words(92, 0, N, K)
    s4 = np.full((N, K // 128), 1.0, np.float16)
    r = synth.int8_uniform(92, 1, (K,))
    r[r == -128] = -127
    r[5] = -127                                 # the largest magnitude is negative
    x = r.astype(np.float16)
    y, xq, sx = _run(Wc, s4, x)
    assert sx[0] == 1.0
    assert_bits_equal(xq, r.astype(np.int8), "codes")
    y_ref, _ = oracle.gemv_w4a8(Wc, s4, r.astype(np.int8), np.float32(1.0))
    assert np.array_equal(y.astype(np.float64), y_ref)


def test_rounding_ties_to_even():
    """s_x = 1 and activations on half-integers: the codes round to even."""
    say("w4a8 ties")
    K = 256
    x = np.zeros(K, np.float16)
    x[0] = 127
    halves = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -126.5], np.float16)
    x[1:1 + halves.size] = halves
    Wc = synth.w4_words(93, 0, 16, K)
    s4 = synth.f16_uniform(93, 1, (16, K // 128), 0.002, 0.02)
    _, xq, sx = _run(Wc, s4, x)
    assert sx[0] == 1.0
    assert xq[1:1 + halves.size].tolist() == [0, 2, 2, 0, -2, -2, 126, -126]
    _check(Wc, s4, x, what="ties")


def test_zero_activation():
    """max |x| = 0 (including -0): s_x = 0, codes 0, y = 0."""
    say("w4a8 zero x")
    N, K = 64, 512
    Wc = synth.w4_words(94, 0, N, K)
    s4 = synth.f16_uniform(94, 1, (N, K // 128), 0.002, 0.02)
    x = np.zeros(K, np.float16)
    x[::3] = np.float16(-0.0)
    y, xq, sx = _run(Wc, s4, x)
    assert sx[0] == 0.0 and not xq.any() and not y.any()


def test_tiny_and_large_activations():
    """Activations near the fp16 extremes: subnormals and 65504."""
    say("w4a8 extreme x")
    N, K = 48, 1024
    Wc = synth.w4_words(95, 0, N, K)
    s4 = synth.f16_uniform(95, 1, (N, K // 128), 0.002, 0.02)
    for scale in (1e-7, 6e-5, 40000.0):
        x = (synth.f16_normal(95, 2, (K,), 1.0).astype(np.float64) * scale / 4).astype(np.float16)
        _check(Wc, s4, x, what=f"scale {scale}")
    x = np.zeros(K, np.float16)
    x[7] = np.float16(65504)
    x[100] = np.float16(-65504)
    x[200] = np.float16(2.0 ** -24)             # smallest subnormal: code 0
    _check(Wc, s4, x, what="65504")


def test_codes_equal_without_outputs():
    """Requesting the codes and scale does not change y."""
    say("w4a8 y without xq_out")
    Wc, s4, x = _case(700, 2048, workload=96)
    Wp, Sp = wsgemv.pack_w4(dev(Wc), dev(s4))
    y0 = host(wsgemv.gemv_w4a8(Wp, Sp, dev(x), 700))
    y1, _, _ = _run(Wc, s4, x)
    assert_bits_equal(y0, y1, "with and without code outputs")


def test_lmhead_full():
    """The full 248320 x 1024 lm_head in int4 with int8 activations."""
    say("w4a8 lm_head 248320x1024")
    N, K = synth.LMHEAD
    Wc, s4, x = _case(N, K, workload=97)
    _check(Wc, s4, x, what="lm_head")


def test_step_with_w4a8_linears():
    """W4A8 linears in a decode step beside W4A16 ones, in both plans."""
    say("step with w4a8")
    lins, checks = [], []
    for i, (N, K) in enumerate([(200, 3072), (1024, 1024), (17, 256)]):
        Wc, s4, x = _case(N, K, workload=98, ids=(3 * i, 3 * i + 1, 3 * i + 2))
        Wp, Sp = wsgemv.pack_w4(dev(Wc), dev(s4))
        y = torch.empty(N, device="cuda")
        lins.append(wsgemv.Linear(wsgemv.W4A8, Wp, dev(x), y, N, K, scale=Sp, group=128))
        xq, sx = oracle.quantize_x_i8(x)
        checks.append((y, *oracle.gemv_w4a8(Wc, s4, xq, sx)))
    Wc, s4, x = _case(500, 2048, workload=98, ids=(20, 21, 22))
    Wp, Sp = wsgemv.pack_w4(dev(Wc), dev(s4))
    y = torch.empty(500, device="cuda")
    lins.append(wsgemv.Linear(wsgemv.W4A16, Wp, dev(x), y, 500, 2048, scale=Sp, group=128))
    checks.append((y, *oracle.gemv_w4a16(Wc, s4, x)))
    outs = {}
    for mode in (wsgemv.STEP_ORDERED, wsgemv.STEP_GROUPED | wsgemv.STEP_FORCE_GRAPH, wsgemv.STEP_GROUPED | wsgemv.STEP_EAGER):
        for yt, _, _ in checks:
            yt.fill_(float("nan"))
        step = wsgemv.DecodeStep(lins, mode)
        step()
        step()
        for yt, y_ref, A in checks:
            assert_within(host(yt), y_ref, A, f"mode {mode:#x}")
        outs[mode] = [host(yt).copy() for yt, _, _ in checks]
        step.close()
    for a, b in zip(outs[wsgemv.STEP_GROUPED | wsgemv.STEP_FORCE_GRAPH], outs[wsgemv.STEP_GROUPED | wsgemv.STEP_EAGER]):
        assert_bits_equal(a, b, "grouped graph vs eager")
