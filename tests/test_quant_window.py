"""The in-kernel per-token int8 quantiser takes the quotient x / s as
fp32(x * fp32(1 / s)) and falls back to the IEEE fp32 division only when that
product lies within 8u|t| (u = 2^-24) of a half-integer.  This checks, in
numpy fp32 arithmetic (IEEE, round to nearest even), that the rule gives the
same codes as clamp(rint(fp32(x / s)), -127, 127) for every finite fp16 input
and a spread of scales s = fp32(max|x|) / 127, including power-of-two scales
whose quotients land exactly on half-integers.  CPU only."""
import numpy as np

U = np.float32(2.0 ** -24)


def codes_division(x, s):
    return np.clip(np.rint(x / s), -127, 127).astype(np.int32)


def codes_window(x, s):
    rs = np.float32(1) / s
    t = (x * rs).astype(np.float32)
    r = np.rint(t)
    dist = np.float32(0.5) - np.abs((t - r).astype(np.float32))
    exact = ~(dist > (np.abs(t) * np.float32(2.0 ** -21)))
    c = np.clip(r, -127, 127).astype(np.int32)
    c[exact] = codes_division(x[exact], s)
    return c, int(exact.sum())


def all_finite_f16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bits.view(np.float16)
    return v[np.isfinite(v)].astype(np.float32)


def test_window_rule_equals_ieee_division():
    x = all_finite_f16()
    rng = np.random.default_rng(7)
    amaxes = np.concatenate([
        rng.choice(np.abs(x[x != 0]), 200, replace=False),                 # random fp16 magnitudes
        np.float32(127.0) * np.float32(2.0) ** np.arange(-20, 9, dtype=np.float32),  # s = 2^k: exact ties
        np.array([65504.0, 2.0 ** -24, 1.0, 127.0, 254.0], dtype=np.float32),
    ]).astype(np.float32)
    fallbacks = plain_misses = 0
    for amax in amaxes:
        s = np.float32(amax) / np.float32(127)
        xs = x[np.abs(x) <= amax]  # values of a vector whose largest magnitude is amax
        want = codes_division(xs, s)
        got, n = codes_window(xs, s)
        fallbacks += n
        assert np.array_equal(got, want), f"amax {amax}: {np.flatnonzero(got != want)[:5]}"
        plain = np.clip(np.rint(xs * (np.float32(1) / s)), -127, 127).astype(np.int32)
        plain_misses += int((plain != want).sum())
    assert fallbacks > 0  # the ties of the power-of-two scales take the division
    assert plain_misses > 0  # the reciprocal alone would miss codes: the window is needed
