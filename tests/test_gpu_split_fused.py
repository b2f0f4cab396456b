"""Split-K summed by the last unit of each row tile, the default for every
kind (fp16, int8 and int4 weights), checked against the same split summed
by the reduce kernel and against the oracle.

Both paths add the S partials in slice order 0..S-1, so they must agree bit
for bit; each is also within the oracle's GEMV bound (int8 accumulators
exactly).  Every call must leave the arrival counters zero, since the next
call relies on it: the workspace is read back after each call.  Repeated
calls with new inputs, the greedy token over a fused split, and a
graph-replayed ORDERED step with split linears are covered too.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_bits_equal, assert_within, dev, host, say
from weight_streaming_gemv_decode_amd import synth, wsgemv

pytestmark = pytest.mark.gpu


def _ctr_off(kind, N, S):
    """Byte offset of the arrival counters in a split workspace."""
    part = S * N * 4 + (256 if kind == wsgemv.W8A8_DYN else 0)
    return (part + 255) // 256 * 256


def _splits(kind, N, K, splits):
    return splits or wsgemv.plan_splits(kind, 1, N, K)


class _Reduce:
    """The reduce-kernel path for the duration of a with-block."""

    def __enter__(self):
        wsgemv.tune_set("split_fuse", 0)

    def __exit__(self, *exc):
        wsgemv.tune_set("split_fuse", -1)


def _counters_zero(ws, kind, N, S, what):
    if ws is None:
        return
    c = host(ws[_ctr_off(kind, N, S):])
    assert c.size >= 4 and not c.any(), f"{what}: arrival counters not zero after the call"


F16_CASES = [(1000, 2048, 2), (248, 4096, 3), (4, 1024, 2), (513, 8192, 0), (128, 8192, 0), (2000, 1024, 7)]


@pytest.mark.parametrize("N,K,splits", F16_CASES)
def test_f16_fused_equals_reduce(N, K, splits):
    S = _splits(wsgemv.F16, N, K, splits)
    assert S > 1
    say(f"fused split f16 {N}x{K} S={S}")
    W = synth.f16_normal(190, N, (N, K), 0.02)
    Wd = dev(W)
    ws = wsgemv.workspace(wsgemv.F16, 1, N, K, splits)
    with _Reduce():
        ws_r = wsgemv.workspace(wsgemv.F16, 1, N, K, splits)
    for rep in range(3):
        x = synth.f16_normal(191, rep, (K,), 1.0)
        y = torch.full((N,), float("nan"), device="cuda")
        wsgemv.gemv_f16(Wd, dev(x), y=y, splits=splits, ws=ws)
        _counters_zero(ws, wsgemv.F16, N, S, f"rep {rep}")
        with _Reduce():
            y_r = wsgemv.gemv_f16(Wd, dev(x), splits=splits, ws=ws_r)
        assert_bits_equal(host(y), host(y_r), f"{N}x{K} S={S} rep {rep}: fused vs reduce kernel")
        assert_within(host(y), *oracle.gemv_f16(W, x), f"{N}x{K} S={S} rep {rep}")


@pytest.mark.parametrize("N,K,splits", [(1000, 4096, 2), (300, 14336, 0), (77, 2048, 5)])
def test_w8a8_fused_equals_reduce(N, K, splits):
    S = _splits(wsgemv.W8A8, N, K, splits)
    assert S > 1
    say(f"fused split w8a8 {N}x{K} S={S}")
    Wq = synth.int8_uniform(192, N, (N, K))
    sw = synth.f32_uniform(192, 1, (N,), 0.001, 0.01)
    ws = wsgemv.workspace(wsgemv.W8A8, 1, N, K, splits)
    for rep in range(2):
        xq = synth.int8_uniform(193, rep, (K,))
        xs = np.array([synth.X_SCALE_W8A8], np.float32)
        y, acc = wsgemv.gemv_w8a8(dev(Wq), dev(sw), dev(xq), dev(xs), splits=splits, ws=ws)
        _counters_zero(ws, wsgemv.W8A8, N, S, f"rep {rep}")
        with _Reduce():
            y_r, acc_r = wsgemv.gemv_w8a8(dev(Wq), dev(sw), dev(xq), dev(xs), splits=splits)
        acc_ref, y_ref, A = oracle.gemv_w8a8(Wq, sw, xq, synth.X_SCALE_W8A8)
        assert_bits_equal(host(acc), acc_ref, f"w8a8 {N}x{K} S={S} rep {rep} accumulators")
        assert_bits_equal(host(y), host(y_r), f"w8a8 {N}x{K} S={S} rep {rep}: fused vs reduce kernel")
        assert_within(host(y), y_ref, A, f"w8a8 {N}x{K} S={S} rep {rep}")


@pytest.mark.parametrize("N,K,splits", [(512, 14336, 0), (256, 8192, 0), (300, 7168, 3)])
def test_w8a8_dyn_fused(N, K, splits):
    """The last unit uses the activation scale it computed itself."""
    S = _splits(wsgemv.W8A8_DYN, N, K, splits)
    assert S > 1
    say(f"fused split w8a8 dyn {N}x{K} S={S}")
    Wq = synth.int8_uniform(194, N, (N, K))
    sw = synth.f32_uniform(194, 1, (N,), 0.001, 0.01)
    ws = wsgemv.workspace(wsgemv.W8A8_DYN, 1, N, K, splits)
    for rep in range(2):
        x = synth.f16_normal(195, rep, (K,), 1.0 + rep)
        acc = torch.empty(N, dtype=torch.int32, device="cuda")
        y = wsgemv.gemv_w8a8_dyn(dev(Wq), dev(sw), dev(x), acc_out=acc, splits=splits, ws=ws)
        _counters_zero(ws, wsgemv.W8A8_DYN, N, S, f"rep {rep}")
        with _Reduce():
            y_r = wsgemv.gemv_w8a8_dyn(dev(Wq), dev(sw), dev(x), splits=splits)
        xq_ref, sx_ref = oracle.quantize_x_i8(x)
        acc_ref, y_ref, A = oracle.gemv_w8a8(Wq, sw, xq_ref, sx_ref)
        assert_bits_equal(host(acc), acc_ref, f"dyn {N}x{K} S={S} rep {rep} accumulators")
        assert_bits_equal(host(y), host(y_r), f"dyn {N}x{K} S={S} rep {rep}: fused vs reduce kernel")
        assert_within(host(y), y_ref, A, f"dyn {N}x{K} S={S} rep {rep}")


@pytest.mark.parametrize("N,K,splits", [(50000, 1024, 2), (777, 4096, 3)])
def test_token_over_fused_split(N, K, splits):
    """The greedy token: one key per row tile, published by the tile's last
    unit; the token is the lowest index of the largest logit the kernel
    wrote, and the same as the reduce path's."""
    say(f"fused split token {N}x{K} S={splits}")
    W = synth.f16_normal(196, N, (N, K), 0.02)
    x = synth.f16_normal(196, 1, (K,), 1.0)
    ws = wsgemv.workspace(wsgemv.F16 | wsgemv.WITH_ARGMAX, 1, N, K, splits)
    y, tok = wsgemv.gemv_f16_argmax(dev(W), dev(x), splits=splits, ws=ws)
    y_h = host(y)
    assert int(host(tok)[0]) == oracle.argmax_f32(y_h)
    with _Reduce():
        y_r, tok_r = wsgemv.gemv_f16_argmax(dev(W), dev(x), splits=splits)
    assert_bits_equal(y_h, host(y_r), "logits: fused vs reduce kernel")
    assert int(host(tok)[0]) == int(host(tok_r)[0])
    y_ref, A = oracle.gemv_f16(W, x)
    assert_within(y_h, y_ref, A, "logits")
    assert oracle.argmax_is_valid(int(host(tok)[0]), y_ref, A)


def test_ordered_step_with_fused_splits_replayed():
    """An ORDERED step (graph-replayed) with split fp16 and int8 linears and
    a token on a split head; four replays with new inputs, each against the
    oracle and bit for bit against the same step planned with the reduce
    kernel."""
    say("ordered step with fused splits, replays")
    shapes = [(512, 8192, 2), (300, 4096, 3), (4000, 2048, 2)]
    Ws = [synth.f16_normal(197, i, (N, K), 0.02) for i, (N, K, _) in enumerate(shapes)]
    Wq = synth.int8_uniform(197, 9, (256, 8192))
    sw = synth.f32_uniform(197, 10, (256,), 0.001, 0.01)
    xs = [torch.empty(K, dtype=torch.float16, device="cuda") for _, K, _ in shapes]
    xq = torch.empty(8192, dtype=torch.int8, device="cuda")
    xsc = dev(np.array([synth.X_SCALE_W8A8], np.float32))

    def plan():
        ys = [torch.empty(N, device="cuda") for N, _, _ in shapes] + [torch.empty(256, device="cuda")]
        tok = torch.empty(1, dtype=torch.int32, device="cuda")
        lins = [wsgemv.Linear(wsgemv.F16, dev(W), x, y, N, K, splits=S,
                              argmax_idx=tok if i == 2 else None)
                for i, ((N, K, S), W, x, y) in enumerate(zip(shapes, Ws, xs, ys))]
        lins.append(wsgemv.Linear(wsgemv.W8A8, dev(Wq), xq, ys[-1], 256, 8192, scale=dev(sw), x_scale=xsc,
                                  splits=4))
        return wsgemv.DecodeStep(lins, wsgemv.STEP_ORDERED | wsgemv.STEP_FORCE_GRAPH), ys, tok

    fused, ys, tok = plan()
    with _Reduce():
        red, ys_r, tok_r = plan()
    assert fused.info()[0] < red.info()[0]           # no reduce launches
    for rep in range(4):
        xin = [synth.f16_normal(198, 10 * rep + i, (K,), 1.0) for i, (_, K, _) in enumerate(shapes)]
        xqi = synth.int8_uniform(198, 10 * rep + 9, (8192,))
        for x, v in zip(xs, xin):
            x.copy_(torch.from_numpy(v))
        xq.copy_(torch.from_numpy(xqi))
        for y in ys + ys_r:
            y.fill_(float("nan"))
        fused()
        red()
        torch.cuda.synchronize()
        for i, (W, v) in enumerate(zip(Ws, xin)):
            assert_bits_equal(host(ys[i]), host(ys_r[i]), f"replay {rep} linear {i}: fused vs reduce kernel")
            assert_within(host(ys[i]), *oracle.gemv_f16(W, v), f"replay {rep} linear {i}")
        _, y_ref, A = oracle.gemv_w8a8(Wq, sw, xqi, synth.X_SCALE_W8A8)
        assert_within(host(ys[-1]), y_ref, A, f"replay {rep} int8")
        assert_bits_equal(host(ys[-1]), host(ys_r[-1]), f"replay {rep} int8: fused vs reduce kernel")
        assert int(host(tok)[0]) == oracle.argmax_f32(host(ys[2]))
        assert int(host(tok)[0]) == int(host(tok_r)[0])
    fused.close()
    red.close()


def _w4(seed, N, K):
    Wc = synth.w4_words(seed, 0, N, K)
    s4 = synth.f16_uniform(seed, 1, (N, K // 128), 0.002, 0.02)
    Wp, Sp = wsgemv.pack_w4(dev(Wc), dev(s4))
    return Wc, s4, Wp, Sp


def _w4_ctr_off(M, N, S):
    return (S * M * N * 4 + 255) // 256 * 256


@pytest.mark.parametrize("M,N,K,splits", [(1, 700, 4096, 2), (1, 64, 8192, 0), (4, 300, 3072, 3), (8, 1000, 2048, 2),
                                          (4, 40, 4096, 0)])
def test_w4a16_fused_equals_reduce(M, N, K, splits):
    S = splits or wsgemv.plan_splits(wsgemv.W4A16, M, N, K)
    assert S > 1
    say(f"fused split w4a16 M={M} {N}x{K} S={S}")
    Wc, s4, Wp, Sp = _w4(199, N, K)
    ws = wsgemv.workspace(wsgemv.W4A16, M, N, K, splits)
    for rep in range(2):
        X = synth.f16_normal(200, rep, (M, K), 1.0)
        y = wsgemv.gemv_w4a16(Wp, Sp, dev(X), N, splits=splits, ws=ws)
        c = host(ws[_w4_ctr_off(M, N, S):])
        assert not c.any(), "arrival counters not zero after the call"
        with _Reduce():
            y_r = wsgemv.gemv_w4a16(Wp, Sp, dev(X), N, splits=splits)
        assert_bits_equal(host(y), host(y_r), f"w4a16 M={M} S={S} rep {rep}: fused vs reduce kernel")
        Y, A = oracle.gemv_w4a16(Wc, s4, X)
        assert_within(host(y).reshape(M, N), Y, A, f"w4a16 M={M} S={S} rep {rep}")


@pytest.mark.parametrize("N,K,splits", [(500, 4096, 2), (48, 8192, 0)])
def test_w4a8_fused_equals_reduce(N, K, splits):
    S = splits or wsgemv.plan_splits(wsgemv.W4A8, 1, N, K)
    assert S > 1
    say(f"fused split w4a8 {N}x{K} S={S}")
    Wc, s4, Wp, Sp = _w4(201, N, K)
    ws = wsgemv.workspace(wsgemv.W4A8, 1, N, K, splits)
    x = synth.f16_normal(202, 0, (K,), 1.0)
    y = wsgemv.gemv_w4a8(Wp, Sp, dev(x), N, splits=splits, ws=ws)
    assert not host(ws[_w4_ctr_off(1, N, S):]).any()
    with _Reduce():
        y_r = wsgemv.gemv_w4a8(Wp, Sp, dev(x), N, splits=splits)
    assert_bits_equal(host(y), host(y_r), "w4a8: fused vs reduce kernel")
    xq, sx = oracle.quantize_x_i8(x)
    assert_within(host(y), *oracle.gemv_w4a8(Wc, s4, xq, sx), "w4a8")


def test_ordered_step_with_fused_w4_split_and_token():
    """An ORDERED step with a split int4 verify block (M = 4) that takes the
    greedy token of every row, replayed: tokens from the tile keys the last
    units publish, equal to the reduce plan's."""
    say("ordered step with a fused int4 split and tokens")
    M, N, K = 4, 5000, 2048
    Wc, s4, Wp, Sp = _w4(203, N, K)
    X = torch.empty((M, K), dtype=torch.float16, device="cuda")

    def plan():
        y = torch.empty((M, N), device="cuda")
        tok = torch.empty(M, dtype=torch.int32, device="cuda")
        lin = wsgemv.Linear(wsgemv.W4A16, Wp, X, y, N, K, M=M, scale=Sp, group=128, splits=2, argmax_idx=tok)
        return wsgemv.DecodeStep([lin], wsgemv.STEP_ORDERED | wsgemv.STEP_FORCE_GRAPH), y, tok

    fused, y, tok = plan()
    with _Reduce():
        red, y_r, tok_r = plan()
    for rep in range(3):
        Xh = synth.f16_normal(204, rep, (M, K), 1.0)
        X.copy_(torch.from_numpy(Xh))
        fused()
        red()
        torch.cuda.synchronize()
        assert_bits_equal(host(y), host(y_r), f"replay {rep}: fused vs reduce kernel")
        Y, A = oracle.gemv_w4a16(Wc, s4, Xh)
        assert_within(host(y), Y, A, f"replay {rep}")
        yh = host(y)
        for m in range(M):
            assert int(host(tok)[m]) == oracle.argmax_f32(yh[m]), f"replay {rep} row {m}"
        assert_bits_equal(host(tok), host(tok_r), f"replay {rep} tokens")
    fused.close()
    red.close()
