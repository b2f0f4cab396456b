"""The CPU oracle against its pins (exact sums, closed forms, numpy, golden
fixtures).  CPU only."""
import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)


def test_thread_count_invariance(orc):
    """Rows are split over threads; every result is bit-identical."""
    import numpy as np
    from weight_streaming_gemv_decode_amd import synth
    W = synth.f16_normal(907, 0, (257, 1024), synth.W_SIGMA)
    x = synth.f16_normal(907, 1, (1024,), synth.X_SIGMA)
    n0 = oracle.max_threads(orc)
    try:
        oracle.set_threads(1, orc)
        y1, a1 = oracle.gemv_f16(W, x, lib=orc)
        oracle.set_threads(max(2, n0), orc)
        y2, a2 = oracle.gemv_f16(W, x, lib=orc)
    finally:
        oracle.set_threads(n0, orc)
    assert np.array_equal(y1, y2) and np.array_equal(a1, a2)


def test_bound_helper():
    import numpy as np
    A = np.array([0.0, 1.0, 1000.0])
    y = np.zeros(3)
    assert oracle.max_err_ratio(y + [1e-6, 1e-3 + 1e-6, 1.0 + 1e-6], y, A) <= 1.0 + 1e-12
    assert oracle.max_err_ratio(y + [3e-6, 0, 0], y, A) > 1.0
    assert oracle.max_err_ratio(y + [float("nan"), 0, 0], y, A) == float("inf")
