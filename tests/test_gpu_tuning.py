"""Every instantiated kernel shape, reached through the launch-table
overrides, returns the same bits as the default shape (only the split-K
slicing may change the summation order, and it is held fixed here) and
stays within the oracle's bound."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_bits_equal, assert_within, dev, host, say
from weight_streaming_gemv_decode_amd import synth, wsgemv

pytestmark = pytest.mark.gpu

KEYS = ("nt", "dense_R", "dense_CH", "dense_rows", "group_R", "group_CH", "group_unit_kb", "w4_R", "w4_B",
        "w4_tiles", "group_w4_tiles", "w4_mfma_m1")


def _pair(kr, kc, R, CH):
    """Set a (rows, vectors) kernel shape; clear both first so no unbuilt
    intermediate pair is ever formed."""
    wsgemv.tune_set(kr, -1)
    wsgemv.tune_set(kc, -1)
    wsgemv.tune_set(kr, R)
    wsgemv.tune_set(kc, CH)


@pytest.fixture(autouse=True)
def _reset():
    for k in KEYS:
        wsgemv.tune_set(k, -1)
    yield
    for k in KEYS:
        wsgemv.tune_set(k, -1)


DENSE_SHAPES = [(4, 2), (2, 2), (1, 2), (8, 1), (4, 1)]


@pytest.mark.parametrize("N,K", [(301, 1024), (77, 1000), (130, 3072)])
@pytest.mark.parametrize("S", [1, 2])
def test_dense_f16_shapes(N, K, S):
    say(f"tuning f16 {N}x{K} S={S}")
    W = synth.f16_normal(80, N, (N, K), synth.W_SIGMA)
    x = synth.f16_normal(80, K, (K,), synth.X_SIGMA)
    y_ref, A = oracle.gemv_f16(W, x)
    Wd, xd = dev(W), dev(x)
    base = host(wsgemv.gemv_f16(Wd, xd, splits=S))
    assert_within(base, y_ref, A, "default")
    for nt in (0, 1):
        for R, CH in DENSE_SHAPES:
            for rows in (R, 4 * R, 5 * R):
                wsgemv.tune_set("nt", nt)
                _pair("dense_R", "dense_CH", R, CH)
                wsgemv.tune_set("dense_rows", rows)
                assert_bits_equal(host(wsgemv.gemv_f16(Wd, xd, splits=S)), base, f"nt={nt} R={R} CH={CH} rows={rows}")


@pytest.mark.parametrize("N,K", [(150, 4096), (33, 2064)])
def test_dense_w8a8_shapes(N, K):
    say(f"tuning w8a8 {N}x{K}")
    Wq = synth.int8_uniform(81, 0, (N, K))
    xq = synth.int8_uniform(81, 1, (K,))
    sw = synth.f32_uniform(81, 2, (N,), 0.001, 0.01)
    acc_ref, y_ref, A = oracle.gemv_w8a8(Wq, sw, xq, 0.02)
    xs = torch.tensor([0.02], device="cuda")
    Wd, xd, sd = dev(Wq), dev(xq), dev(sw)
    for S in (1, 3):
        y0, a0 = wsgemv.gemv_w8a8(Wd, sd, xd, xs, splits=S)
        y0, a0 = host(y0), host(a0)
        assert_bits_equal(a0, acc_ref, f"S={S} acc")
        assert_within(y0, y_ref, A, f"S={S}")
        for R, CH in DENSE_SHAPES:
            _pair("dense_R", "dense_CH", R, CH)
            wsgemv.tune_set("dense_rows", 2 * R)
            y, a = wsgemv.gemv_w8a8(Wd, sd, xd, xs, splits=S)
            assert_bits_equal(host(a), acc_ref, f"R={R} CH={CH} acc")
            assert_bits_equal(host(y), y0, f"R={R} CH={CH} y")


@pytest.mark.parametrize("M", [1, 4])
@pytest.mark.parametrize("N,K", [(100, 1024), (40, 3072), (17, 640)])
def test_w4_shapes(M, N, K):
    say(f"tuning w4 M={M} {N}x{K}")
    Wc = synth.w4_words(82, N, N, K)
    s4 = synth.f16_uniform(82, K, (N, K // 128), 0.002, 0.02)
    X = synth.f16_normal(82, M, (M, K), synth.X_SIGMA)
    Y_ref, A = oracle.gemv_w4a16(Wc, s4, X)
    Wp, Sp = wsgemv.pack_w4(dev(Wc), dev(s4))
    Xd = dev(X)
    base = host(wsgemv.gemv_w4a16(Wp, Sp, Xd, N, splits=1))
    assert_within(base, Y_ref, A, "default")
    for nt in (0, 1):
        for R in (1, 2):
            for B in (4, 8):
                for tiles in (1, 3):
                    wsgemv.tune_set("nt", nt)
                    wsgemv.tune_set("w4_R", R)
                    wsgemv.tune_set("w4_B", B)
                    wsgemv.tune_set("w4_tiles", tiles)
                    got = host(wsgemv.gemv_w4a16(Wp, Sp, Xd, N, splits=1))
                    assert_bits_equal(got, base, f"nt={nt} R={R} B={B} tiles={tiles}")


@pytest.mark.parametrize("N,K", [(100, 1024), (17, 640)])
def test_w4_m1_on_matrix_cores(N, K):
    """M = 1 through the matrix-core kernel (a tuning switch): a different
    summation order, so within the bound rather than bit-identical, and
    every shape of that kernel bit-identical to its own default."""
    say(f"tuning w4 M=1 on MFMA {N}x{K}")
    Wc = synth.w4_words(83, N, N, K)
    s4 = synth.f16_uniform(83, K, (N, K // 128), 0.002, 0.02)
    x = synth.f16_normal(83, 1, (K,), synth.X_SIGMA)
    y_ref, A = oracle.gemv_w4a16(Wc, s4, x)
    Wp, Sp = wsgemv.pack_w4(dev(Wc), dev(s4))
    wsgemv.tune_set("w4_mfma_m1", 1)
    base = host(wsgemv.gemv_w4a16(Wp, Sp, dev(x), N, splits=1))
    assert_within(base, y_ref.reshape(N), A.reshape(N), "mfma M=1")
    for R, B in ((1, 4), (2, 4), (1, 8)):
        wsgemv.tune_set("w4_R", R)
        wsgemv.tune_set("w4_B", B)
        got = host(wsgemv.gemv_w4a16(Wp, Sp, dev(x), N, splits=1))
        assert_bits_equal(got, base, f"mfma M=1 R={R} B={B}")


def test_grouped_shapes_bit_identical():
    say("tuning grouped step shapes")
    step = synth.decode_step_f16(workload=83, n_layers=1, lm_head_rows=4000)
    lins = []
    for name, W, x in step:
        N, K = W.shape
        lins.append(wsgemv.Linear(wsgemv.F16, dev(W), dev(x), torch.empty(N, device="cuda"), N, K))
    st = wsgemv.DecodeStep(lins, wsgemv.STEP_GROUPED)
    st()
    base = [host(l.y).copy() for l in lins]
    st.close()
    for (name, W, x), b in zip(step, base):
        y_ref, A = oracle.gemv_f16(W, x)
        assert_within(b, y_ref, A, name)
    for R, CH in ((4, 2), (2, 2), (8, 1)):
        for kb in (16, 64, 300):
            _pair("group_R", "group_CH", R, CH)
            wsgemv.tune_set("group_unit_kb", kb)
            st = wsgemv.DecodeStep(lins, wsgemv.STEP_GROUPED)
            st()
            for l, b in zip(lins, base):
                assert_bits_equal(host(l.y), b, f"grouped R={R} CH={CH} unit={kb}KB")
            st.close()


@pytest.mark.parametrize("N,K", [(100, 1024), (40, 3072), (17, 640)])
def test_w4a8_shapes(N, K):
    """Every int8-activation kernel shape returns the default's bits, codes and scale."""
    say(f"tuning w4a8 {N}x{K}")
    Wc = synth.w4_words(84, N, N, K)
    s4 = synth.f16_uniform(84, K, (N, K // 128), 0.002, 0.02)
    x = synth.f16_normal(84, 1, (K,), synth.X_SIGMA)
    xq_ref, sx_ref = oracle.quantize_x_i8(x)
    y_ref, A = oracle.gemv_w4a8(Wc, s4, xq_ref, sx_ref)
    Wp, Sp = wsgemv.pack_w4(dev(Wc), dev(s4))
    xd = dev(x)
    base = host(wsgemv.gemv_w4a8(Wp, Sp, xd, N, splits=1))
    assert_within(base, y_ref, A, "default")
    xq = torch.empty(K, dtype=torch.int8, device="cuda")
    sx = torch.empty(1, device="cuda")
    for nt in (0, 1):
        for R in (1, 2):
            for B in (4, 8):
                for tiles in (1, 3):
                    wsgemv.tune_set("nt", nt)
                    wsgemv.tune_set("w4_R", R)
                    wsgemv.tune_set("w4_B", B)
                    wsgemv.tune_set("w4_tiles", tiles)
                    xq.fill_(99)
                    sx.fill_(float("nan"))
                    got = host(wsgemv.gemv_w4a8(Wp, Sp, xd, N, xq_out=xq, sx_out=sx, splits=1))
                    what = f"nt={nt} R={R} B={B} tiles={tiles}"
                    assert_bits_equal(got, base, what)
                    assert_bits_equal(host(xq), xq_ref, what + " codes")
                    assert_bits_equal(host(sx), np.array([sx_ref], np.float32), what + " scale")


def test_grouped_w4_shapes_bit_identical():
    """Grouped int4 steps (fp16 and int8 activations) at every kernel shape."""
    say("tuning grouped w4 step shapes")
    lins, refs = [], []
    for i, (N, K) in enumerate([(200, 3072), (1024, 1024), (17, 256), (333, 640)]):
        Wc = synth.w4_words(85, 3 * i, N, K)
        s4 = synth.f16_uniform(85, 3 * i + 1, (N, K // 128), 0.002, 0.02)
        x = synth.f16_normal(85, 3 * i + 2, (K,), synth.X_SIGMA)
        Wp, Sp = wsgemv.pack_w4(dev(Wc), dev(s4))
        for kind in (wsgemv.W4A16, wsgemv.W4A8):
            lins.append(wsgemv.Linear(kind, Wp, dev(x), torch.empty(N, device="cuda"), N, K, scale=Sp, group=128))
            if kind == wsgemv.W4A8:
                refs.append(oracle.gemv_w4a8(Wc, s4, *oracle.quantize_x_i8(x)))
            else:
                refs.append(oracle.gemv_w4a16(Wc, s4, x))
    st = wsgemv.DecodeStep(lins, wsgemv.STEP_GROUPED)
    st()
    base = [host(l.y).copy() for l in lins]
    st.close()
    for b, (y_ref, A) in zip(base, refs):
        assert_within(b, y_ref, A, "grouped default")
    for R in (1, 2):
        for B in (4, 8):
            for tiles in (1, 2, 8, 16):
                wsgemv.tune_set("w4_R", R)
                wsgemv.tune_set("w4_B", B)
                wsgemv.tune_set("group_w4_tiles", tiles)
                st = wsgemv.DecodeStep(lins, wsgemv.STEP_GROUPED)
                st()
                for l, b in zip(lins, base):
                    assert_bits_equal(host(l.y), b, f"grouped w4 R={R} B={B} tiles={tiles}")
                st.close()
