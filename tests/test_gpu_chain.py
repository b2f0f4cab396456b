"""Dependent linears: each linear's fp16 output copy (y16) is the next
linear's input, run by the ORDERED plan.

The exact case uses signed permutation matrices scaled by powers of two, in
fp16 and in int4 (q - 8 = +-1 with a power-of-two group scale): every
product, sum and rounding is exact, so every stage of the GPU chain must
equal the oracle chain bit for bit; a stage that ran early or read a stale
input could not.  The random case keeps each stage within the GEMV bound
plus the propagated effect of the previous stages' bounds and roundings,
all computed from the oracle's own chain."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_bits_equal, dev, host, say
from weight_streaming_gemv_decode_amd import synth, wsgemv

pytestmark = pytest.mark.gpu


def _w4_signed_perm(N, K, perm, sign, j):
    """Canonical int4 words and fp16 scales holding sign * 2^j at (n, perm[n])."""
    q = np.full((N, K), 8, np.uint32)
    q[np.arange(N), perm] = (8 + sign).astype(np.uint32)
    words = np.zeros((N, K // 8), np.uint32)
    for i in range(8):
        words |= q[:, i::8] << np.uint32(4 * i)
    s4 = np.full((N, K // 128), 2.0 ** j, np.float16)
    return words, s4


def _abs_w4(words, s4):
    """|w| = |q - 8| * s of canonical int4 words (for the propagated bound)."""
    N, K8 = words.shape
    q = np.empty((N, K8 * 8), np.int64)
    for i in range(8):
        q[:, i::8] = (words >> np.uint32(4 * i)) & np.uint32(15)
    return np.abs(q - 8) * np.repeat(s4.astype(np.float64), 128, axis=1)


def _oracle_stage(kind, W, x):
    if kind == wsgemv.F16:
        y, A = oracle.gemv_f16(W[0], x)
    else:
        y, A = oracle.gemv_w4a16(W[0], W[1], x)
    return y.reshape(-1), A.reshape(-1)


def _build(stages, x0, splits=()):
    """Linears of the chain on the GPU: stage i reads stage i-1's y16."""
    lins, y16s, ys = [], [], []
    x = dev(x0)
    for i, (kind, W, N, K) in enumerate(stages):
        y = torch.empty(N, device="cuda")
        y16 = torch.empty(N, dtype=torch.float16, device="cuda")
        s = 2 if i in splits else 0
        if kind == wsgemv.F16:
            lin = wsgemv.Linear(wsgemv.F16, dev(W[0]), x[:K], y, N, K, splits=s, y16=y16)
        else:
            Wp, Sp = wsgemv.pack_w4(dev(W[0]), dev(W[1]))
            lin = wsgemv.Linear(wsgemv.W4A16, Wp, x[:K], y, N, K, scale=Sp, group=128, splits=s, y16=y16)
        lins.append(lin)
        ys.append(y)
        y16s.append(y16)
        x = y16
    return lins, ys, y16s


@pytest.mark.parametrize("mode", [wsgemv.STEP_ORDERED, wsgemv.STEP_ORDERED | wsgemv.STEP_FORCE_GRAPH])
@pytest.mark.parametrize("split", [False, True])
def test_exact_chain(mode, split):
    say(f"chain exact mode={mode:#x} split={split}")
    K, depth = 1024, 8
    r = synth.rng(160, 0)
    # small integers: 8 stages of factors 2^-1..2^1 stay exact and finite in fp16
    x0 = r.integers(-64, 65, K).astype(np.float16)
    stages = []
    for i in range(depth):
        perm, sign, j = r.permutation(K), r.choice([-1, 1], K), int(r.integers(-1, 2))
        if i % 2 == 0:
            W = np.zeros((K, K), np.float16)
            W[np.arange(K), perm] = sign * 2.0 ** j
            stages.append((wsgemv.F16, (W,), K, K))
        else:
            stages.append((wsgemv.W4A16, _w4_signed_perm(K, K, perm, sign, j), K, K))
    lins, ys, y16s = _build(stages, x0, splits=(1, 2, 5) if split else ())
    step = wsgemv.DecodeStep(lins, mode)
    for rep in range(2):
        for y16 in y16s:
            y16.fill_(float("nan"))
        step()
        x = x0
        for i, (kind, W, N, K_) in enumerate(stages):
            y_ref, _ = _oracle_stage(kind, W, x[:K_])
            x = oracle.round_f16(y_ref)
            assert_bits_equal(host(ys[i]).astype(np.float64), y_ref, f"stage {i} y, replay {rep}")
            assert_bits_equal(host(y16s[i]), x, f"stage {i} y16, replay {rep}")
    step.close()


def _ulp16(v):
    """Spacing of fp16 values at magnitude v (the subnormal spacing below 2^-14)."""
    v = np.maximum(np.abs(np.asarray(v, np.float64)), 2.0 ** -14)
    return 2.0 ** (np.floor(np.log2(v)) - 10)


@pytest.mark.parametrize("mode", [wsgemv.STEP_ORDERED, wsgemv.STEP_ORDERED | wsgemv.STEP_EAGER])
def test_random_chain_within_propagated_bound(mode):
    """Decode-layer shapes chained through prefixes of y16 (2048 -> 1024,
    6144 -> 3072), fp16 and int4 stages, unit-gain weights."""
    say(f"chain random mode={mode:#x}")
    shapes = [(wsgemv.F16, 2048, 1024), (wsgemv.W4A16, 1024, 1024), (wsgemv.F16, 6144, 1024),
              (wsgemv.W4A16, 1024, 3072), (wsgemv.F16, 2048, 1024), (wsgemv.F16, 1024, 1024)]
    stages = []
    for i, (kind, N, K) in enumerate(shapes):
        if kind == wsgemv.F16:
            stages.append((kind, (synth.f16_normal(161, i, (N, K), 1.0 / np.sqrt(K)),), N, K))
        else:
            Wc = synth.w4_words(161, 100 + i, N, K)
            # |q - 8| averages 4.0, so this scale gives unit gain
            s4 = (synth.f16_uniform(161, 200 + i, (N, K // 128), 0.5, 1.5).astype(np.float64)
                  / (4.6 * np.sqrt(K))).astype(np.float16)
            stages.append((kind, (Wc, s4), N, K))
    x0 = synth.f16_normal(162, 0, (1024,), synth.X_SIGMA)
    lins, ys, y16s = _build(stages, x0, splits=(3,))
    step = wsgemv.DecodeStep(lins, mode)
    step()
    x = x0.astype(np.float16)
    tol_x = np.zeros(x.size)                    # bound on |x_gpu - x_oracle|, per element
    for i, (kind, W, N, K) in enumerate(stages):
        y_ref, A = _oracle_stage(kind, W, x[:K])
        absW = np.abs(W[0].astype(np.float64)) if kind == wsgemv.F16 else _abs_w4(W[0], W[1])
        tol = oracle.bound(A) + 1.001 * (absW @ tol_x[:K])
        y = host(ys[i]).astype(np.float64)
        err = np.abs(y - y_ref)
        assert np.all(np.isfinite(y)) and np.all(err <= tol), \
            f"stage {i}: max err / tol = {float(np.max(err / tol)):.3g}"
        # the kernel's own rounding of its fp32 output, against numpy's
        assert_bits_equal(host(y16s[i]), host(ys[i]).astype(np.float16), f"stage {i} y16")
        # the next input: the oracle's rounding; the two roundings differ by at
        # most the inputs' difference plus one fp16 spacing
        x = oracle.round_f16(y_ref)
        tol_x = tol + _ulp16(np.abs(y_ref) + tol)
    step.close()


def test_y16_with_k_zero_and_grouped():
    """K = 0 writes y16 = 0; a GROUPED plan of independent linears writes
    each y16 as its y rounded."""
    say("y16 K=0 and grouped")
    yz = torch.full((64,), 5.0, device="cuda")
    y16z = torch.full((64,), 5.0, dtype=torch.float16, device="cuda")
    lins = [wsgemv.Linear(wsgemv.F16, torch.empty((64, 0), dtype=torch.float16, device="cuda"),
                          torch.empty(0, dtype=torch.float16, device="cuda"), yz, 64, 0, y16=y16z)]
    W = synth.f16_normal(163, 0, (300, 1024), synth.W_SIGMA)
    x = synth.f16_normal(163, 1, (1024,), synth.X_SIGMA)
    y = torch.empty(300, device="cuda")
    y16 = torch.empty(300, dtype=torch.float16, device="cuda")
    lins.append(wsgemv.Linear(wsgemv.F16, dev(W), dev(x), y, 300, 1024, y16=y16))
    Wc = synth.w4_words(163, 2, 200, 1024)
    s4 = synth.f16_uniform(163, 3, (200, 8), 0.002, 0.02)
    Wp, Sp = wsgemv.pack_w4(dev(Wc), dev(s4))
    X = synth.f16_normal(163, 4, (4, 1024), synth.X_SIGMA)
    Y = torch.empty((4, 200), device="cuda")
    Y16 = torch.empty((4, 200), dtype=torch.float16, device="cuda")
    lins.append(wsgemv.Linear(wsgemv.W4A16, Wp, dev(X), Y, 200, 1024, M=4, scale=Sp, group=128, y16=Y16))
    step = wsgemv.DecodeStep(lins, wsgemv.STEP_GROUPED)
    step()
    assert np.all(host(y16z) == 0) and np.all(host(yz) == 0)
    assert_bits_equal(host(y16), host(y).astype(np.float16), "fp16 linear y16")
    assert_bits_equal(host(Y16), host(Y).astype(np.float16), "verify block y16")
    step.close()
