"""INT4 (W4A16) GEMV on the GPU: load-time packing plus the fused-dequant
kernels, at M = 1 (VALU) and at a verify block M = 2..8 (MFMA)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_bits_equal, assert_within, dev, host, say
from weight_streaming_gemv_decode_amd import synth, wsgemv

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _case(M, N, K, workload=5, ids=(0, 1, 2)):
    Wc = synth.w4_words(workload, ids[0], N, K)
    s4 = synth.f16_uniform(workload, ids[1], (N, K // 128), 0.002, 0.02)
    X = synth.f16_normal(workload, ids[2], (M, K), synth.X_SIGMA)
    return Wc, s4, X


def _gpu(Wc, s4, X, splits=0):
    N = Wc.shape[0]
    Wp, Sp = wsgemv.pack_w4(dev(Wc), dev(s4))
    return host(wsgemv.gemv_w4a16(Wp, Sp, dev(X), N, splits=splits))


def test_golden_nibble_order_through_pack_and_kernel():
    say("w4 golden nibble order")
    g = json.load(open(os.path.join(GOLDEN, "w4_nibble_order.json")))
    K = g["K"]
    rows = g["rows"]
    N = len(rows)
    Wc = np.zeros((N, K // 8), np.uint32)
    s4 = np.zeros((N, 1), np.uint16)
    for n, r in enumerate(rows):
        Wc[n, :] = int(r["rest"], 16)
        Wc[n, 0] = int(r["word0"], 16)
        s4[n, 0] = int(r["scale_bits"], 16)
    X = np.zeros((8, K), np.float16)
    X[np.arange(8), np.arange(8)] = 1           # row m is e_m: a verify block of 8
    Wp, Sp = wsgemv.pack_w4(dev(Wc), dev(s4.view(np.float16)))
    for M in (1, 8):
        y = host(wsgemv.gemv_w4a16(Wp, Sp, dev(X[:M]), N))
        y = y.reshape(M, N)
        for n, r in enumerate(rows):
            assert y[:, n].tolist() == r["y_onehot_j0_to_7"][:M], (M, n, y[:, n])


@pytest.mark.parametrize("N,K", [(1, 128), (16, 128), (17, 256), (100, 640), (2048, 1024), (1024, 3072),
                                 (33, 4096), (5, 8192)])
def test_m1_shapes(N, K):
    say(f"w4 M=1 {N}x{K}")
    Wc, s4, X = _case(1, N, K, workload=70, ids=(N, K, N + K))
    y_ref, A = oracle.gemv_w4a16(Wc, s4, X)
    y = _gpu(Wc, s4, X)
    assert_within(y.reshape(1, N), y_ref, A, f"{N}x{K}")


@pytest.mark.parametrize("S", [1, 2, 3, 6])
def test_m1_splits(S):
    N, K = 1024, 3072
    say(f"w4 M=1 {N}x{K} S={S}")
    Wc, s4, X = _case(1, N, K)
    y_ref, A = oracle.gemv_w4a16(Wc, s4, X)
    y = _gpu(Wc, s4, X, splits=S)
    assert_within(y.reshape(1, N), y_ref, A, f"S={S}")


@pytest.mark.parametrize("M", [2, 3, 4, 5, 8])
@pytest.mark.parametrize("N,K", [(64, 1024), (200, 3072), (17, 256)])
def test_mfma_block(M, N, K):
    say(f"w4 M={M} {N}x{K}")
    Wc, s4, X = _case(M, N, K, workload=71, ids=(M, N, K))
    Y_ref, A = oracle.gemv_w4a16(Wc, s4, X)
    Y = _gpu(Wc, s4, X)
    assert_within(Y, Y_ref, A, f"M={M} {N}x{K}")


@pytest.mark.parametrize("S", [2, 3])
def test_mfma_splits(S):
    M, N, K = 4, 512, 3072
    say(f"w4 M={M} S={S}")
    Wc, s4, X = _case(M, N, K, workload=72)
    Y_ref, A = oracle.gemv_w4a16(Wc, s4, X)
    assert_within(_gpu(Wc, s4, X, splits=S), Y_ref, A, f"M=4 S={S}")


def test_verify_block_identical_rows():
    say("w4 M=4 identical rows")
    Wc, s4, X = _case(1, 300, 1024, workload=73)
    Xr = np.repeat(X, 4, axis=0)
    Y = _gpu(Wc, s4, Xr)
    for m in range(1, 4):
        assert_bits_equal(Y[m], Y[0], f"row {m} vs row 0")
    y_ref, A = oracle.gemv_w4a16(Wc, s4, X)
    assert_within(Y[:1], y_ref, A, "M=4 row 0")


@pytest.mark.parametrize("name,N,K", [(s.name, s.N, s.K) for s in synth.DECODE_LAYER] +
                         [("lm_head", synth.LMHEAD[0], synth.LMHEAD[1])])
@pytest.mark.parametrize("M", [1, 4])
def test_decode_shapes(name, N, K, M):
    say(f"w4 {name} {N}x{K} M={M}")
    tid = sum(map(ord, name))
    Wc, s4, X = _case(M, N, K, workload=5, ids=(tid, 500 + tid, 2000 + M))
    Y_ref, A = oracle.gemv_w4a16(Wc, s4, X)
    assert_within(_gpu(Wc, s4, X), Y_ref, A, f"{name} M={M}")


def test_degenerate():
    say("w4 N=0, K=0")
    y = torch.full((2, 3), 4.0, device="cuda")
    wsgemv.gemv_w4a16(torch.empty(16, dtype=torch.uint8, device="cuda"),
                      torch.empty(16, dtype=torch.uint8, device="cuda"),
                      torch.empty((2, 0), dtype=torch.float16, device="cuda"), 3, y=y)
    assert host(y).tolist() == [[0.0] * 3] * 2
