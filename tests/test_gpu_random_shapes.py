"""Seeded random shapes for every kind, against the oracle.

The fixed-shape tests pin the tile edges the kernels were written for; these
draw N anywhere in 1..6000 (every ragged tail of a row tile and of a work
unit), K any multiple of the kind's vector width, M 1..8 for int4 verify
blocks, and splits 0 (the launch table's choice), 1, 2, 3 or 5.  A draw
whose split would leave a k-slice empty or exceed a slice's limit must be
refused with WSG_ERR_SHAPE (the rules of include/wsgemv.h, restated below);
every other draw must match the oracle: int32 accumulators and int8 codes
bit for bit, fp results within 1e-3 A + 1e-6.  Two mixed decode steps
(GROUPED and ORDERED) over random kinds and shapes check every linear the
same way."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_bits_equal, assert_within, dev, host, say
from weight_streaming_gemv_decode_amd import synth, wsgemv

pytestmark = pytest.mark.gpu

SHAPE = 2
SPLITS = (0, 0, 1, 2, 3, 5)


def _cdiv(a, b):
    return -(-a // b)


def _dense_split_ok(kvec, S):
    """Dense kinds: a forced split is whole vectors per slice, at most 2048
    of them, and leaves no slice empty."""
    if S == 0:
        return True
    return S <= kvec and _cdiv(kvec, S) <= 2048 and (S - 1) * _cdiv(kvec, S) < kvec


def _w4_split_ok(M, kb, S):
    """int4 kinds: slices are whole 4-block quads, none empty, and M rows of
    a slice's activations fit the 48 KiB stage."""
    if S == 0:
        return True
    if S > kb:
        return False
    if S == 1:
        return M * kb * 256 <= 48 * 1024
    kbs = _cdiv(_cdiv(kb, S), 4) * 4
    return (S - 1) * kbs < kb and M * kbs * 256 <= 48 * 1024


def _draws(seed, n, kmax, kunit, mmax=1):
    r = synth.rng(191, seed)
    out = []
    for i in range(n):
        N = int(r.integers(1, 6001))
        K = kunit * int(r.integers(1, kmax // kunit + 1))
        M = int(r.integers(1, mmax + 1))
        S = int(r.choice(SPLITS))
        out.append((i, M, N, K, S))
    return out


def _expect_refused(fn, what):
    with pytest.raises(wsgemv.WsgError) as e:
        fn()
    assert e.value.status == SHAPE, (what, e.value.status)


@pytest.mark.parametrize("i,M,N,K,S", _draws(0, 30, 4096, 8))
def test_f16(i, M, N, K, S):
    what = f"f16 #{i} {N}x{K} S={S}"
    say(what)
    W = synth.f16_normal(192, 2 * i, (N, K), synth.W_SIGMA)
    x = synth.f16_normal(192, 2 * i + 1, (K,), synth.X_SIGMA)
    ws = lambda: wsgemv.workspace(wsgemv.F16, 1, N, K, S)  # noqa: E731
    if not _dense_split_ok(K // 8, S):
        _expect_refused(lambda: wsgemv.gemv_f16(dev(W), dev(x), splits=S, ws=ws()), what)
        return
    y = host(wsgemv.gemv_f16(dev(W), dev(x), splits=S, ws=ws()))
    y_ref, A = oracle.gemv_f16(W, x)
    assert_within(y, y_ref, A, what)


@pytest.mark.parametrize("i,M,N,K,S", _draws(1, 20, 8192, 16))
def test_w8a8(i, M, N, K, S):
    what = f"w8a8 #{i} {N}x{K} S={S}"
    say(what)
    Wq = synth.int8_uniform(193, 3 * i, (N, K))
    sw = synth.f32_uniform(193, 3 * i + 1, (N,), 0.001, 0.01)
    xq = synth.int8_uniform(193, 3 * i + 2, (K,))
    xs = torch.tensor([synth.X_SCALE_W8A8], device="cuda")
    ws = lambda: wsgemv.workspace(wsgemv.W8A8, 1, N, K, S)  # noqa: E731
    if not _dense_split_ok(K // 16, S):
        _expect_refused(lambda: wsgemv.gemv_w8a8(dev(Wq), dev(sw), dev(xq), xs, splits=S, ws=ws()), what)
        return
    y, acc = wsgemv.gemv_w8a8(dev(Wq), dev(sw), dev(xq), xs, splits=S, ws=ws())
    acc_ref, y_ref, A = oracle.gemv_w8a8(Wq, sw, xq, synth.X_SCALE_W8A8)
    assert_bits_equal(host(acc), acc_ref, f"{what} accumulators")
    assert_within(host(y), y_ref, A, what)


@pytest.mark.parametrize("i,M,N,K,S", _draws(2, 20, 16384, 16))
def test_w8a8_dyn(i, M, N, K, S):
    what = f"w8a8 dyn #{i} {N}x{K} S={S}"
    say(what)
    Wq = synth.int8_uniform(194, 3 * i, (N, K))
    sw = synth.f32_uniform(194, 3 * i + 1, (N,), 0.001, 0.01)
    x = synth.f16_normal(194, 3 * i + 2, (K,), synth.X_SIGMA)
    ws = lambda: wsgemv.workspace(wsgemv.W8A8_DYN, 1, N, K, S)  # noqa: E731
    if not _dense_split_ok(K // 16, S):
        _expect_refused(lambda: wsgemv.gemv_w8a8_dyn(dev(Wq), dev(sw), dev(x), splits=S, ws=ws()), what)
        return
    acc = torch.empty(N, dtype=torch.int32, device="cuda")
    xq = torch.empty(K, dtype=torch.int8, device="cuda")
    sx = torch.empty(1, device="cuda")
    y = wsgemv.gemv_w8a8_dyn(dev(Wq), dev(sw), dev(x), acc_out=acc, xq_out=xq, sx_out=sx, splits=S, ws=ws())
    xq_ref, sx_ref = oracle.quantize_x_i8(x)
    assert_bits_equal(host(xq), xq_ref, f"{what} codes")
    assert_bits_equal(host(sx), np.array([sx_ref], np.float32), f"{what} scale")
    acc_ref, y_ref, A = oracle.gemv_w8a8(Wq, sw, xq_ref, sx_ref)
    assert_bits_equal(host(acc), acc_ref, f"{what} accumulators")
    assert_within(host(y), y_ref, A, what)


def _w4_case(workload, i, M, N, K):
    Wc = synth.w4_words(workload, 3 * i, N, K)
    s4 = synth.f16_uniform(workload, 3 * i + 1, (N, K // 128), 0.002, 0.02)
    X = synth.f16_normal(workload, 3 * i + 2, (M, K), synth.X_SIGMA)
    return Wc, s4, X


@pytest.mark.parametrize("i,M,N,K,S", _draws(3, 30, 3072, 128, mmax=8))
def test_w4a16(i, M, N, K, S):
    what = f"w4a16 #{i} M={M} {N}x{K} S={S}"
    say(what)
    Wc, s4, X = _w4_case(195, i, M, N, K)
    Wp, Sp = wsgemv.pack_w4(dev(Wc), dev(s4))
    ws = lambda: wsgemv.workspace(wsgemv.W4A16, M, N, K, S)  # noqa: E731
    if not _w4_split_ok(M, K // 128, S):
        _expect_refused(lambda: wsgemv.gemv_w4a16(Wp, Sp, dev(X), N, splits=S, ws=ws()), what)
        return
    y = host(wsgemv.gemv_w4a16(Wp, Sp, dev(X), N, splits=S, ws=ws())).reshape(M, N)
    y_ref, A = oracle.gemv_w4a16(Wc, s4, X)
    assert_within(y, y_ref, A, what)


@pytest.mark.parametrize("i,M,N,K,S", _draws(4, 15, 8192, 128))
def test_w4a8(i, M, N, K, S):
    what = f"w4a8 #{i} {N}x{K} S={S}"
    say(what)
    Wc, s4, X = _w4_case(196, i, 1, N, K)
    x = X.reshape(K)
    Wp, Sp = wsgemv.pack_w4(dev(Wc), dev(s4))
    ws = lambda: wsgemv.workspace(wsgemv.W4A8, 1, N, K, S)  # noqa: E731
    if not _w4_split_ok(1, K // 128, S):
        _expect_refused(lambda: wsgemv.gemv_w4a8(Wp, Sp, dev(x), N, splits=S, ws=ws()), what)
        return
    xq = torch.empty(K, dtype=torch.int8, device="cuda")
    sx = torch.empty(1, device="cuda")
    y = host(wsgemv.gemv_w4a8(Wp, Sp, dev(x), N, xq_out=xq, sx_out=sx, splits=S, ws=ws()))
    xq_ref, sx_ref = oracle.quantize_x_i8(x)
    assert_bits_equal(host(xq), xq_ref, f"{what} codes")
    assert_bits_equal(host(sx), np.array([sx_ref], np.float32), f"{what} scale")
    y_ref, A = oracle.gemv_w4a8(Wc, s4, xq_ref, sx_ref)
    assert_within(y, y_ref, A, what)


@pytest.mark.parametrize("mode", [wsgemv.STEP_GROUPED, wsgemv.STEP_ORDERED])
def test_mixed_decode_step(mode):
    """Twelve linears of random kinds and shapes in one plan (each with its
    own inputs and outputs), two replays; every output against the oracle."""
    say(f"random mixed step mode={mode}")
    r = synth.rng(197, mode)
    lins, checks = [], []
    for i in range(12):
        kind = int(r.choice([wsgemv.F16, wsgemv.W8A8, wsgemv.W8A8_DYN, wsgemv.W4A16, wsgemv.W4A8]))
        N = int(r.integers(1, 4001))
        if kind == wsgemv.F16:
            K = 8 * int(r.integers(1, 385))
            W = synth.f16_normal(198, 4 * i, (N, K), synth.W_SIGMA)
            x = synth.f16_normal(198, 4 * i + 1, (K,), synth.X_SIGMA)
            y = torch.empty(N, device="cuda")
            lins.append(wsgemv.Linear(kind, dev(W), dev(x), y, N, K))
            y_ref, A = oracle.gemv_f16(W, x)
            checks.append((y, y_ref, A, None, None, f"#{i} f16 {N}x{K}"))
        elif kind in (wsgemv.W8A8, wsgemv.W8A8_DYN):
            K = 16 * int(r.integers(1, 257))
            Wq = synth.int8_uniform(198, 4 * i, (N, K))
            sw = synth.f32_uniform(198, 4 * i + 1, (N,), 0.001, 0.01)
            y = torch.empty(N, device="cuda")
            acc = torch.empty(N, dtype=torch.int32, device="cuda")
            if kind == wsgemv.W8A8:
                xq = synth.int8_uniform(198, 4 * i + 2, (K,))
                xs = torch.tensor([synth.X_SCALE_W8A8], device="cuda")
                lins.append(wsgemv.Linear(kind, dev(Wq), dev(xq), y, N, K, scale=dev(sw), x_scale=xs, acc_out=acc))
                acc_ref, y_ref, A = oracle.gemv_w8a8(Wq, sw, xq, synth.X_SCALE_W8A8)
            else:
                x = synth.f16_normal(198, 4 * i + 2, (K,), synth.X_SIGMA)
                lins.append(wsgemv.Linear(kind, dev(Wq), dev(x), y, N, K, scale=dev(sw), acc_out=acc))
                xq_ref, sx_ref = oracle.quantize_x_i8(x)
                acc_ref, y_ref, A = oracle.gemv_w8a8(Wq, sw, xq_ref, sx_ref)
            checks.append((y, y_ref, A, acc, acc_ref, f"#{i} kind {kind} {N}x{K}"))
        else:
            K = 128 * int(r.integers(1, 17))
            M = int(r.integers(1, 9)) if kind == wsgemv.W4A16 else 1
            Wc, s4, X = _w4_case(199, i, M, N, K)
            Wp, Sp = wsgemv.pack_w4(dev(Wc), dev(s4))
            y = torch.empty((M, N) if kind == wsgemv.W4A16 else (N,), device="cuda")
            xin = dev(X) if kind == wsgemv.W4A16 else dev(X.reshape(K))
            lins.append(wsgemv.Linear(kind, Wp, xin, y, N, K, M=M, scale=Sp, group=128))
            if kind == wsgemv.W4A16:
                y_ref, A = oracle.gemv_w4a16(Wc, s4, X)
            else:
                xq_ref, sx_ref = oracle.quantize_x_i8(X.reshape(K))
                y_ref, A = oracle.gemv_w4a8(Wc, s4, xq_ref, sx_ref)
            checks.append((y, y_ref, A, None, None, f"#{i} kind {kind} M={M} {N}x{K}"))
    step = wsgemv.DecodeStep(lins, mode)
    for rep in range(2):
        for y, *_ in checks:
            y.fill_(float("nan"))
        step()
        for y, y_ref, A, acc, acc_ref, what in checks:
            yy = host(y)
            assert_within(yy.reshape(np.shape(y_ref)), y_ref, A, f"replay {rep} {what}")
            if acc is not None:
                assert_bits_equal(host(acc), acc_ref, f"replay {rep} {what} accumulators")
    step.close()
