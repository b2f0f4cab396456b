"""gemv_f16_static (the allocation-free gemv_f16) on the GPU, through the C
ABI: bit for bit equal to gemv_f16 with a caller workspace, over two calls
in a row whose second is smaller (the scratch array keeps the first call's
partials, which the second must not read), at forced and automatic splits;
the lm_head-sized call is also checked against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_bits_equal, assert_within, dev, host, say
from weight_streaming_gemv_decode_amd import synth, wsgemv

pytestmark = pytest.mark.gpu


def _pair(N, K, S, workload):
    W = synth.f16_normal(workload, 0, (N, K), synth.W_SIGMA)
    x = synth.f16_normal(workload, 1, (K,), synth.X_SIGMA)
    Wd, xd = dev(W), dev(x)
    y_ws = host(wsgemv.gemv_f16(Wd, xd, splits=S))
    y_st = torch.full((N,), float("nan"), device="cuda")
    wsgemv.gemv_f16_static(Wd, xd, y_st, splits=S)
    return W, x, y_ws, host(y_st)


@pytest.mark.parametrize("first,second", [((248320, 1024, 2), (5000, 2048, 3)),
                                          ((20000, 3072, 0), (333, 1000, 2))])
def test_static_equals_workspace_path_two_calls(first, second):
    for i, (N, K, S) in enumerate((first, second)):
        say(f"gemv_f16_static call {i}: {N}x{K} S={S}")
        W, x, y_ws, y_st = _pair(N, K, S, workload=70 + i)
        assert wsgemv.plan_splits(0, 1, N, K) >= 1
        assert_bits_equal(y_st, y_ws, f"static vs workspace {N}x{K} S={S}")
        if i == 0 and N == 248320:
            y_ref, A = oracle.gemv_f16(W, x)
            assert_within(y_st, y_ref, A, "lm_head through the static scratch")


def test_static_too_large_is_rejected_and_k_zero():
    say("gemv_f16_static limits")
    # S * N * 4 bytes of partials beyond the scratch array: refused, nothing launched
    N, K, S = 1 << 21, 64, 3
    assert S * N * 4 > wsgemv.STATIC_SCRATCH_BYTES
    W = torch.empty((N, K), dtype=torch.float16, device="cuda")
    x = torch.zeros(K, dtype=torch.float16, device="cuda")
    y = torch.full((N,), 7.0, device="cuda")
    with pytest.raises(wsgemv.WsgError, match="WSG_ERR_WORKSPACE"):
        wsgemv.gemv_f16_static(W, x, y, splits=S)
    torch.cuda.synchronize()
    assert float(y[0]) == 7.0 and float(y[-1]) == 7.0
    del W
    # K = 0 writes y = 0
    y = torch.full((100,), 3.0, device="cuda")
    wsgemv.gemv_f16_static(torch.empty((100, 0), dtype=torch.float16, device="cuda"),
                           torch.empty(0, dtype=torch.float16, device="cuda"), y)
    assert not host(y).any()
