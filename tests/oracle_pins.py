"""Pins of the CPU oracle to facts outside the oracle itself.

Each ``pin_*`` function takes a loaded oracle library and raises
AssertionError when the oracle disagrees with something the mathematics or a
hand-derived fixture fixes: exact rational sums (Python ``fractions``),
numpy's own fp16 conversion and float64 / int64 matrix products on an
independent dequantisation, closed forms (identity, permutation, one-hot,
powers of two), hand-packed int4 words and the exact int32 range boundary.
They are plain functions so that the mutation test can run the same checks
against deliberately broken copies of the oracle.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

import oracle
from weight_streaming_gemv_decode_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U53 = 2.0 ** -53


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bits(a):
    return np.array([[int(v, 16) for v in row] for row in a], dtype=np.uint16) if isinstance(a[0], list) \
        else np.array([int(v, 16) for v in a], dtype=np.uint16)


def _frac16(h: np.ndarray):
    """Exact Fractions of fp16 values, via numpy's own conversion."""
    return [Fraction(float(v)) for v in np.asarray(h, np.float16).astype(np.float64).ravel()]


# ---------------------------------------------------------------- fp16 ---

def pin_f16_decode_all_patterns(lib):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 10) & 31) != 31
    got = oracle.f16_decode(bits[finite], lib=lib)
    ref = bits[finite].view(np.float16).astype(np.float64)
    assert np.array_equal(got.view(np.uint64), ref.view(np.uint64)), "fp16 decode differs from numpy"
    for bad in (0x7C00, 0xFC00, 0x7E00, 0x7C01):
        try:
            oracle.f16_decode(np.array([bad], np.uint16), lib=lib)
        except oracle.OracleError:
            continue
        raise AssertionError(f"Inf/NaN pattern {bad:#06x} not rejected")


def pin_f16_golden(lib):
    g = _golden("f16_tiny.json")
    W, x = _bits(g["W_bits"]), _bits(g["x_bits"])
    y, A = oracle.gemv_f16(W, x, lib=lib)
    assert np.array_equal(y, np.array(g["y"])), (y, g["y"])
    assert np.array_equal(A, np.array(g["A"])), (A, g["A"])


def pin_f16_exact_rational(lib, N=7, K=40, seed=11):
    W = synth.f16_normal(900, seed, (N, K), synth.W_SIGMA)
    x = synth.f16_normal(900, seed + 1, (K,), synth.X_SIGMA)
    W[0, :4] = np.array([2 ** -24, -(2 ** -24), 2 ** -14, 65504], np.float16)   # subnormal / extreme
    y, A = oracle.gemv_f16(W, x, lib=lib)
    xf = _frac16(x)
    for n in range(N):
        wf = _frac16(W[n])
        exact = sum(a * b for a, b in zip(wf, xf))
        absum = sum(abs(a * b) for a, b in zip(wf, xf))
        tol = K * U53 * float(absum)
        assert abs(Fraction(y[n]) - exact) <= Fraction(tol), (n, y[n], float(exact))
        assert abs(Fraction(A[n]) - absum) <= Fraction(tol), (n, A[n], float(absum))


def pin_f16_closed_forms(lib, K=48, seed=12):
    x = synth.f16_normal(901, seed, (K,), synth.X_SIGMA)
    xd = x.astype(np.float64)
    eye = np.eye(K, dtype=np.float16)
    y, _ = oracle.gemv_f16(eye, x, lib=lib)
    assert np.array_equal(y, xd), "identity W must return x exactly"
    perm = np.random.default_rng(5).permutation(K)
    P = np.zeros((K, K), np.float16)
    P[np.arange(K), perm] = 1
    y, _ = oracle.gemv_f16(P, x, lib=lib)
    assert np.array_equal(y, xd[perm]), "permutation W must permute x exactly"
    y, A = oracle.gemv_f16(np.ones((3, K), np.float16), np.ones(K, np.float16), lib=lib)
    assert np.array_equal(y, np.full(3, float(K))) and np.array_equal(A, np.full(3, float(K)))
    # rows 2^j * e_{k(n)}: a rectangular W (N != K), so a transposed operand
    # or a wrong row stride cannot pass
    N = 5
    ks = [3, 0, K - 1, 17, 29]
    Wr = np.zeros((N, K), np.float16)
    for n, k in enumerate(ks):
        Wr[n, k] = np.float16(2.0 ** (n - 2))
    y, _ = oracle.gemv_f16(Wr, x, lib=lib)
    assert np.array_equal(y, np.array([2.0 ** (n - 2) * xd[k] for n, k in enumerate(ks)]))


def pin_f16_numpy_matmul(lib, N=64, K=1000, seed=13):
    W = synth.f16_normal(902, seed, (N, K), synth.W_SIGMA)
    x = synth.f16_normal(902, seed + 1, (K,), synth.X_SIGMA)
    y, A = oracle.gemv_f16(W, x, lib=lib)
    Wd, xd = W.astype(np.float64), x.astype(np.float64)
    ref = Wd @ xd
    refA = np.abs(Wd) @ np.abs(xd)
    assert np.all(np.abs(y - ref) <= 1e-12 * refA), "oracle differs from numpy float64 matmul"
    assert np.all(np.abs(A - refA) <= 1e-12 * refA)


def pin_f16_scaling(lib, N=9, K=64, seed=14):
    W = synth.f16_normal(903, seed, (N, K), synth.W_SIGMA)
    x = synth.f16_normal(903, seed + 1, (K,), synth.X_SIGMA)
    y1, _ = oracle.gemv_f16(W, x, lib=lib)
    y2, _ = oracle.gemv_f16(W, (x.astype(np.float32) * 4).astype(np.float16), lib=lib)
    assert np.array_equal(y2, 4 * y1), "power-of-two scaling of x must scale y exactly"


# ---------------------------------------------------------------- w8a8 ---

def pin_w8a8_golden(lib):
    g = _golden("w8a8_tiny.json")
    acc, y, A = oracle.gemv_w8a8(np.array(g["Wq"], np.int8), np.array(g["w_scale"], np.float32),
                                 np.array(g["xq"], np.int8), g["x_scale"], lib=lib)
    assert acc.tolist() == g["acc"], acc
    assert np.array_equal(y, np.array(g["y"])) and np.array_equal(A, np.array(g["A"])), (y, A)


def pin_w8a8_int64_matmul(lib, N=37, K=300, seed=15):
    Wq = synth.int8_uniform(904, seed, (N, K))
    xq = synth.int8_uniform(904, seed + 1, (K,))
    Wq[0, :5] = -128
    xq[:3] = -128
    s_w = synth.f32_uniform(904, seed + 2, (N,), 0.001, 0.01)
    s_x = np.float32(0.02)
    acc, y, A = oracle.gemv_w8a8(Wq, s_w, xq, s_x, lib=lib)
    ref = Wq.astype(np.int64) @ xq.astype(np.int64)
    assert np.array_equal(acc.astype(np.int64), ref), "int8 accumulator differs from int64 matmul"
    absref = np.abs(Wq.astype(np.int64)) @ np.abs(xq.astype(np.int64))
    for n in range(N):
        sc = Fraction(float(s_w[n])) * Fraction(float(s_x))
        assert abs(Fraction(y[n]) - int(ref[n]) * sc) <= abs(int(ref[n]) * sc) * Fraction(U53)
        assert abs(Fraction(A[n]) - int(absref[n]) * sc) <= abs(int(absref[n]) * sc) * Fraction(U53)
    # one-hot rows select activations; x = 1 gives row sums
    sel = np.random.default_rng(3).integers(0, K, N)
    oh = np.zeros((N, K), np.int8)
    oh[np.arange(N), sel] = 1
    acc1, _, _ = oracle.gemv_w8a8(oh, s_w, xq, s_x, lib=lib)
    assert np.array_equal(acc1, xq[sel].astype(np.int32))
    acc2, _, _ = oracle.gemv_w8a8(Wq, s_w, np.ones(K, np.int8), s_x, lib=lib)
    assert np.array_equal(acc2, Wq.astype(np.int64).sum(1).astype(np.int32))


def pin_w8a8_int32_range(lib):
    one = np.ones(1, np.float32)

    def run(K, w, xv):
        return oracle.gemv_w8a8(np.full((1, K), w, np.int8), one, np.full(K, xv, np.int8), 1.0, lib=lib)

    acc, _, _ = run(133144, 127, 127)               # 133144 * 16129 = 2147479576 <= 2^31 - 1
    assert int(acc[0]) == 133144 * 16129
    acc, _, _ = run(132104, -128, 127)              # -132104 * 16256 = -2147482624 >= -2^31
    assert int(acc[0]) == -132104 * 16256
    for K, w, xv in ((133145, 127, 127), (131072, -128, -128), (132105, -128, 127)):
        try:
            run(K, w, xv)
        except oracle.OracleError as e:
            assert f"status {oracle.ERR_RANGE}" in str(e)
            continue
        raise AssertionError(f"int32 overflow not detected for K={K}")


# ---------------------------------------------------------------- w4a16 --

def _unpack_canonical(Wc: np.ndarray) -> np.ndarray:
    """Independent numpy unpack: q[n, 8j+i] = (Wc[n,j] >> 4i) & 15."""
    shifts = (4 * np.arange(8, dtype=np.uint32))[None, None, :]
    return ((Wc[:, :, None] >> shifts) & np.uint32(15)).reshape(Wc.shape[0], -1).astype(np.int64)


def pin_w4_golden(lib):
    g = _golden("w4_nibble_order.json")
    K, group = g["K"], g["group"]
    for row in g["rows"]:
        Wc = np.full((1, K // 8), int(row["rest"], 16), np.uint32)
        Wc[0, 0] = int(row["word0"], 16)
        s4 = np.array([[int(row["scale_bits"], 16)]], np.uint16)
        for j, want in enumerate(row["y_onehot_j0_to_7"]):
            x = np.zeros(K, np.float16)
            x[j] = 1
            y, _ = oracle.gemv_w4a16(Wc, s4, x, group, lib=lib)
            assert y[0] == want, (row["word0"], j, y[0], want)
    tg = g["two_group_case"]
    K2 = tg["K"]
    s4 = np.array([[int(v, 16) for v in tg["scale_bits"]]], np.uint16)
    for row in tg["rows"]:
        Wc = np.concatenate([np.full(16, int(w, 16), np.uint32) for w in row["group_words"]])[None, :]
        y, _ = oracle.gemv_w4a16(Wc, s4, np.ones(K2, np.float16), group, lib=lib)
        assert y[0] == row["y_all_ones_x"], (row, y[0])


def pin_w4_numpy_dequant(lib, M=3, N=40, K=512, seed=16):
    Wc = synth.w4_words(905, seed, N, K)
    s4 = synth.f16_uniform(905, seed + 1, (N, K // 128), 0.002, 0.02)
    X = synth.f16_normal(905, seed + 2, (M, K), synth.X_SIGMA)
    Y, A = oracle.gemv_w4a16(Wc, s4, X, 128, lib=lib)
    w = (_unpack_canonical(Wc) - 8).astype(np.float64) * np.repeat(s4.astype(np.float64), 128, axis=1)
    ref = X.astype(np.float64) @ w.T
    refA = np.abs(X.astype(np.float64)) @ np.abs(w).T
    assert np.all(np.abs(Y - ref) <= 1e-12 * refA + 1e-300), "w4 oracle differs from numpy dequant+matmul"
    assert np.all(np.abs(A - refA) <= 1e-12 * refA + 1e-300)
    # every row of a block equals the M=1 product of that row, bit for bit
    for m in range(M):
        y1, a1 = oracle.gemv_w4a16(Wc, s4, X[m], 128, lib=lib)
        assert np.array_equal(y1, Y[m]) and np.array_equal(a1, A[m])


def pin_w4_exact_rational(lib, N=3, K=256, seed=17):
    Wc = synth.w4_words(906, seed, N, K)
    s4 = synth.f16_uniform(906, seed + 1, (N, K // 128), 0.002, 0.02)
    x = synth.f16_normal(906, seed + 2, (K,), synth.X_SIGMA)
    y, _ = oracle.gemv_w4a16(Wc, s4, x, 128, lib=lib)
    q = _unpack_canonical(Wc)
    xf = _frac16(x)
    for n in range(N):
        sf = _frac16(s4[n])
        terms = [(int(q[n, k]) - 8) * sf[k // 128] * xf[k] for k in range(K)]
        exact = sum(terms)
        tol = Fraction(K * U53) * sum(abs(t) for t in terms)
        assert abs(Fraction(y[n]) - exact) <= tol, (n, y[n], float(exact))


# ---------------------------------------------------------------- w4a8 ---

def pin_quant_golden(lib):
    g = _golden("w4a8_quant.json")
    for c in g["cases"]:
        xq, sx = oracle.quantize_x_i8(np.array(c["x"], np.float16), lib=lib)
        assert xq.tolist() == c["xq"], (c["x"], xq.tolist(), c["xq"])
        assert float(sx) == c["s_x"], (sx, c["s_x"])


def pin_quant_properties(lib, K=3000, seed=18):
    x = synth.f16_normal(907, seed, (K,), synth.X_SIGMA)
    xq, sx = oracle.quantize_x_i8(x, lib=lib)
    xf = x.astype(np.float32)
    amax = np.max(np.abs(xf))
    assert sx == np.float32(amax) / np.float32(127), "s_x must be fp32 max|x| / 127"
    assert np.all(np.abs(xq.astype(np.int32)) <= 127)
    assert np.all(np.abs(xq[np.abs(xf) == amax].astype(np.int32)) == 127), "max |x| must map to +-127"
    assert np.all(np.sign(xq) == np.sign(np.rint(xf / sx)))
    # round to nearest: every code is within half a step of x / s_x
    assert np.all(np.abs(xf.astype(np.float64) / float(sx) - xq) <= 0.5 + 1e-6)
    # numpy's own IEEE fp32 division and half-to-even rounding give the same codes
    assert np.array_equal(np.clip(np.rint(xf / sx), -127, 127).astype(np.int8), xq)


def pin_w4a8_golden(lib):
    g = _golden("w4_nibble_order.json")
    K = g["K"]
    for row in g["rows"]:
        if row["scale_bits"] != "0x3C00":
            continue
        Wc = np.full((1, K // 8), int(row["rest"], 16), np.uint32)
        Wc[0, 0] = int(row["word0"], 16)
        s4 = np.array([[0x3C00]], np.uint16)
        for j, want in enumerate(row["y_onehot_j0_to_7"]):
            xq = np.zeros(K, np.int8)
            xq[j] = 1
            y, _ = oracle.gemv_w4a8(Wc, s4, xq, 1.0, lib=lib)
            assert y[0] == want, (row["word0"], j, y[0])
            y, _ = oracle.gemv_w4a8(Wc, s4, 3 * xq, 0.5, lib=lib)
            assert y[0] == 1.5 * want


def pin_w4a8_integer_matmul(lib, N=23, K=512, seed=19):
    Wc = synth.w4_words(908, seed, N, K)
    xq = synth.int8_uniform(908, seed + 1, (K,))
    xq[:2] = -127
    ones = np.full((N, K // 128), 0x3C00, np.uint16)
    y, A = oracle.gemv_w4a8(Wc, ones, xq, 1.0, lib=lib)
    w = _unpack_canonical(Wc) - 8
    ref = w @ xq.astype(np.int64)
    assert np.array_equal(y, ref.astype(np.float64)), "unit scales: y must be the exact integer product"
    assert np.array_equal(A, (np.abs(w) @ np.abs(xq.astype(np.int64))).astype(np.float64))
    s4 = synth.f16_uniform(908, seed + 2, (N, K // 128), 0.002, 0.02)
    y2, A2 = oracle.gemv_w4a8(Wc, s4, xq, 0.03125, lib=lib)
    wf = w.astype(np.float64) * np.repeat(s4.astype(np.float64), 128, axis=1)
    ref2 = (wf @ xq.astype(np.float64)) * 0.03125
    assert np.all(np.abs(y2 - ref2) <= 1e-12 * A2 + 1e-300)


# -------------------------------------------------------------- argmax ---

def pin_argmax_golden(lib):
    g = _golden("argmax_ties.json")
    for c in g["cases"]:
        y = np.array([int(v, 16) for v in c["bits"]], np.uint32).view(np.float32)
        assert oracle.argmax_f32(y, lib=lib) == c["argmax"], c["note"]


def pin_argmax_numpy(lib, n=5000, seed=20):
    """numpy's argmax (first occurrence of the maximum; -0 == +0) on finite
    values with many exact ties, and nanargmax where NaNs are present."""
    r = synth.rng(909, seed)
    for trial in range(20):
        y = np.round(r.normal(0, 3, n)).astype(np.float32)      # integers: many ties
        y[r.integers(0, n, 50)] = -0.0
        assert oracle.argmax_f32(y, lib=lib) == int(np.argmax(y)), trial
        y[r.integers(0, n, 200)] = np.nan
        assert oracle.argmax_f32(y, lib=lib) == int(np.nanargmax(y)), trial
    y = np.zeros(n, np.float32)
    y[-1] = 1
    assert oracle.argmax_f32(y, lib=lib) == n - 1


def pin_topk_golden(lib):
    g = _golden("topk_order.json")
    for c in g["cases"]:
        y = np.array([int(v, 16) for v in c["bits"]], np.uint32).view(np.float32)
        assert oracle.topk_f32(y, c["k"], lib=lib).tolist() == c["topk"], c["note"]


def pin_topk_numpy(lib, n=3000, seed=25):
    """numpy's stable lexicographic sort on (-value, index) puts NaN last and
    keeps equal values (and -0 / +0) in index order: its first k entries are
    the top-k; k = 1 is the greedy token."""
    r = synth.rng(914, seed)
    for trial in range(10):
        y = np.round(r.normal(0, 4, n)).astype(np.float32)
        y[r.integers(0, n, 40)] = -0.0
        if trial % 2:
            y[r.integers(0, n, 100)] = np.nan
        want = np.lexsort((np.arange(n), -y))
        for k in (1, 7, 64, n):
            got = oracle.topk_f32(y, k, lib=lib)
            assert np.array_equal(got, want[:k]), (trial, k)
        assert int(oracle.topk_f32(y, 1, lib=lib)[0]) == oracle.argmax_f32(y, lib=lib)


# ---------------------------------------------------------- fp16 chain ---

def pin_round_f16_golden(lib):
    """Hand-derived binary16 roundings: ties go to the even significand."""
    cases = [(1.0, 0x3C00), (-0.0, 0x8000), (65504.0, 0x7BFF), (65519.99, 0x7BFF), (65520.0, 0x7C00),
             (-1e6, 0xFC00), (2.0 ** -24, 0x0001), (2.0 ** -25, 0x0000), (3 * 2.0 ** -25, 0x0002),
             (2.0 ** -14, 0x0400), (1 + 2.0 ** -11, 0x3C00), (1 + 3 * 2.0 ** -11, 0x3C02),
             (2049.0, 0x6800), (2051.0, 0x6802), (0.1, 0x2E66), (-2.5, 0xC100)]
    got = oracle.round_f16(np.array([c[0] for c in cases]), lib=lib).view(np.uint16)
    for (v, want), g in zip(cases, got):
        assert int(g) == want, (v, hex(int(g)), hex(want))


def pin_round_f16_numpy(lib, seed=21):
    """numpy's own float64 -> float16 cast, including exact midpoints."""
    r = synth.rng(910, seed)
    h = r.integers(0, 0x7BFF, 20000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    v = np.concatenate([r.normal(0, 1, 20000), r.normal(0, 1e4, 5000), r.normal(0, 1e-6, 5000),
                        (lo + hi) / 2, -(lo + hi) / 2])
    with np.errstate(over="ignore"):
        want = v.astype(np.float16)
    assert np.array_equal(oracle.round_f16(v, lib=lib).view(np.uint16), want.view(np.uint16))


def pin_chain_permutations(lib, K=256, depth=5, seed=22):
    """Signed permutation matrices times 2^j: every fp16 value is exact, so
    the chain's output is the input permuted, signed and scaled."""
    r = synth.rng(911, seed)
    x = r.integers(-1000, 1000, K).astype(np.float16)
    Ws, want = [], x.astype(np.float64)
    for i in range(depth):
        perm = r.permutation(K)
        sign = r.choice([-1.0, 1.0], K)
        j = int(r.integers(-2, 3))
        W = np.zeros((K, K), np.float16)
        W[np.arange(K), perm] = sign * 2.0 ** j
        Ws.append(W)
        want = sign * 2.0 ** j * want[perm]
    out = oracle.chain_f16(Ws, x, lib=lib)
    assert np.array_equal(out[-1][0], want)
    assert np.array_equal(out[-1][1].astype(np.float64), want)


# ----------------------------------------------------- causal conv1d ---

def pin_conv_golden(lib):
    g = _golden("conv1d_step.json")
    for c in g["cases"]:
        w = np.array(c["w"], np.float16)
        b = None if c["bias"] is None else np.array(c["bias"], np.float32)
        out, A, st = oracle.causal_conv1d_step(np.array(c["x"], np.float32), w, b,
                                               np.array(c["state"], np.float32), c["silu"], lib=lib)
        assert np.allclose(out, c["out"], rtol=1e-15, atol=1e-15), (out, c["out"])
        assert st.tolist() == c["new_state"]


def pin_conv_sequence_numpy(lib, C=37, W=4, T=12, seed=23):
    """T steps from a zero state equal numpy's correlation of each channel's
    whole input history with its taps (y_t = sum_j w[j] x[t - W + 1 + j])."""
    r = synth.rng(912, seed)
    w = r.normal(0, 0.5, (C, W)).astype(np.float16)
    b = r.normal(0, 1, C).astype(np.float32)
    xs = r.normal(0, 1, (T, C)).astype(np.float32)
    st = np.zeros((C, W - 1), np.float32)
    for t in range(T):
        out, A, st = oracle.causal_conv1d_step(xs[t], w, b, st, False, lib=lib)
        hist = np.concatenate([np.zeros((W - 1, C)), xs[:t + 1].astype(np.float64)])  # zero history first
        for c in range(C):
            want = np.correlate(hist[-W:, c], w[c].astype(np.float64), mode="valid")[0] + float(b[c])
            assert abs(out[c] - want) <= 1e-12 * (A[c] + 1), (t, c, out[c], want)
        assert np.array_equal(st, hist[-(W - 1):].T.astype(np.float32)), t  # the last W - 1 inputs
    # SiLU is x * sigmoid(x) on the same pre-activation
    out_s, _, _ = oracle.causal_conv1d_step(xs[0], w, b, st, True, lib=lib)
    pre, _, _ = oracle.causal_conv1d_step(xs[0], w, b, st, False, lib=lib)
    assert np.allclose(out_s, pre / (1 + np.exp(-pre)), rtol=1e-14, atol=1e-300)


def pin_conv_special_kernels(lib, C=16, W=3, seed=24):
    """Tap W-1 only: out = x exactly; tap 0 only: out = the input W-1 steps ago."""
    r = synth.rng(913, seed)
    xs = r.normal(0, 1, (6, C)).astype(np.float32)
    last = np.zeros((C, W), np.float16)
    last[:, W - 1] = 1
    first = np.zeros((C, W), np.float16)
    first[:, 0] = 1
    st1 = np.zeros((C, W - 1), np.float32)
    st2 = st1.copy()
    for t in range(6):
        o1, _, st1 = oracle.causal_conv1d_step(xs[t], last, None, st1, False, lib=lib)
        o2, _, st2 = oracle.causal_conv1d_step(xs[t], first, None, st2, False, lib=lib)
        assert np.array_equal(o1, xs[t].astype(np.float64))
        assert np.array_equal(o2, xs[t - W + 1].astype(np.float64) if t >= W - 1 else np.zeros(C))


ALL_PINS = [
    pin_f16_decode_all_patterns, pin_f16_golden, pin_f16_exact_rational, pin_f16_closed_forms,
    pin_f16_numpy_matmul, pin_f16_scaling, pin_w8a8_golden, pin_w8a8_int64_matmul,
    pin_w8a8_int32_range, pin_w4_golden, pin_w4_numpy_dequant, pin_w4_exact_rational,
    pin_quant_golden, pin_quant_properties, pin_w4a8_golden, pin_w4a8_integer_matmul,
    pin_argmax_golden, pin_argmax_numpy, pin_round_f16_golden, pin_round_f16_numpy, pin_chain_permutations,
    pin_conv_golden, pin_conv_sequence_numpy, pin_conv_special_kernels, pin_topk_golden, pin_topk_numpy,
]
