"""Plants plausible mistakes in copies of the oracle (on the CPU) and checks
that the pins catch every one of them.  The real oracle is never modified."""
import os
import shutil

import pytest

import oracle
from tests import oracle_pins

# (name, unique text in oracle.c, replacement); every mutant stays in bounds.
MUTANTS = [
    ("f16_drop_last_term", "double p = w * xd[k];", "double p = (k == K - 1) ? 0.0 : w * xd[k];"),
    ("f16_reversed_k", "f16_value(row[k], &w)", "f16_value(row[K - 1 - k], &w)"),
    ("f16_abs_x", "double p = w * xd[k];", "double p = w * fabs(xd[k]);"),
    ("f16_exponent_bias", "(int)e - 25", "(int)e - 24"),
    ("f16_subnormal_scale", "ldexp((double)m, -24)", "ldexp((double)m, -25)"),
    ("f16_sign_dropped", "*out = sign ? -v : v;", "*out = v;"),
    ("f16_A_without_abs", "            a += fabs(p);\n        }\n        y[n] = s;",
     "            a += p;\n        }\n        y[n] = s;"),
    ("w8_unsigned_weight", "(int64_t)row[k] * (int64_t)xq[k]", "(int64_t)(uint8_t)row[k] * (int64_t)xq[k]"),
    ("w8_drop_first_term", "(int64_t)row[k] * (int64_t)xq[k];", "(int64_t)row[k] * (int64_t)xq[k] * (k != 0);"),
    ("w8_no_range_check", "if (s > INT32_MAX || s < INT32_MIN)", "if (0)"),
    ("w8_scale_missing_x", "(double)w_scale[n] * (double)x_scale", "(double)w_scale[n]"),
    ("w4_nibble_order", "(word >> (4 * (k % 8)))", "(word >> (4 * (7 - k % 8)))"),
    ("w4_zero_point", "double w = (double)(q - 8) * scale;", "double w = (double)(q - 7) * scale;"),
    ("w4_group_index", "s4[n * groups + k / group]", "s4[n * groups + (k / 8) % groups]"),
    ("w4a8_group_index", "s4[n * groups + (k / group)]", "s4[n * groups + (k / 8) % groups]"),
    ("w4_activation_row", "w * xd[m * K + k]", "w * xd[k]"),
    ("quant_ties_away", "float r = rintf(t);", "float r = roundf(t);"),
    ("quant_truncate", "float r = rintf(t);", "float r = truncf(t);"),
    ("quant_signed_max", "float a = fabsf((float)v);", "float a = (float)v;"),
    ("quant_scale_255", "volatile float s = amax / 127.0f;", "volatile float s = amax / 255.0f;"),
    ("w4a8_zero_point", "double p = (double)(q - 8) * scale * (double)xq[k];",
     "double p = (double)(q - 7) * scale * (double)xq[k];"),
    ("w4a8_no_sx", "y[n] = s * (double)s_x;", "y[n] = s;"),
    ("argmax_ties_last", "if (isnan(y[best]) || y[i] > y[best])", "if (isnan(y[best]) || y[i] >= y[best])"),
    ("argmax_nan_above", "        if (isnan(y[i]))\n            continue;\n", ""),
    ("argmax_nan_first", "if (isnan(y[best]) || y[i] > y[best])", "if (y[i] > y[best])"),
    ("argmax_skip_last", "for (int64_t i = 1; i < n; ++i) {", "for (int64_t i = 1; i < n - 1; ++i) {"),
    ("round_ties_away", "double r = nearbyint(q);", "double r = round(q);"),
    ("round_truncate", "double r = nearbyint(q);", "double r = trunc(q);"),
    ("round_overflow_early", "if (mag >= 65520.0 || isinf(a))", "if (mag >= 65504.0 || isinf(a))"),
    ("round_no_subnormal_grid", "        e = -14;\n", "        e = -24;\n"),
    ("round_exponent_bias", "(me - 1 + 15) << 10", "(me + 15) << 10"),
    ("conv_taps_reversed", "f16_value(w[c * W + j], &wv)", "f16_value(w[c * W + (W - 1 - j)], &wv)"),
    ("conv_shift_wrong_way", "state[c * (W - 1) + j] = state[c * (W - 1) + j + 1];",
     "state[c * (W - 1) + j + 1] = state[c * (W - 1) + j];"),
    ("conv_no_bias", "double pre = bias ? (double)bias[c] : 0.0;", "double pre = 0.0;"),
    ("conv_silu_sign", "pre / (1.0 + exp(-pre))", "pre / (1.0 + exp(pre))"),
    ("conv_x_not_appended", "state[c * (W - 1) + W - 2] = x[c];", "state[c * (W - 1) + W - 2] = 0.0f;"),
    ("topk_ties_reversed", "    return a < b;\n}", "    return a > b;\n}"),
    ("topk_nan_first", "        return nb;                      /* the number comes before the NaN */",
     "        return na;"),
    ("topk_ascending", "        return va > vb;", "        return va < vb;"),
    ("argmax_signed_zero", "if (isnan(y[best]) || y[i] > y[best])",
     "if (isnan(y[best]) || y[i] > y[best] || (y[i] == y[best] && signbit(y[best]) && !signbit(y[i])))"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} must be unique"
    mdir = tmp_path / "oracle"
    mdir.mkdir()
    (mdir / "oracle.c").write_text(src.replace(old, new))
    so = str(mdir / "liboracle.so")
    import subprocess
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-std=c99", "-shared", "-fPIC",
                    str(mdir / "oracle.c"), "-o", so, "-lm"], check=True)
    lib = oracle.load(so)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, oracle.OracleError):
            caught.append(pin.__name__)
    assert caught, f"no pin detects mutant {name}"
