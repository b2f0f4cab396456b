"""fp16 GEMV (M = 1) on the GPU against the CPU oracle: the 2048x2048 case,
the ~248k-row lm_head with split-K partials reduced on the device, ragged
shapes, the degenerate sizes and exact invariants."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_bits_equal, assert_within, dev, host, say
from weight_streaming_gemv_decode_amd import synth, wsgemv

pytestmark = pytest.mark.gpu


def _case(N, K, workload=1, w_id=0, x_id=1):
    W = synth.f16_normal(workload, w_id, (N, K), synth.W_SIGMA)
    x = synth.f16_normal(workload, x_id, (K,), synth.X_SIGMA)
    return W, x


def test_c1_2048x2048_auto_split():
    N, K = synth.C1_SHAPE
    say(f"f16 C1 {N}x{K} auto")
    W, x = _case(N, K)
    y_ref, A = oracle.gemv_f16(W, x)
    y = host(wsgemv.gemv_f16(dev(W), dev(x)))
    assert_within(y, y_ref, A, "C1")


@pytest.mark.parametrize("S", [1, 2, 3, 4])
def test_c1_split_invariance_and_determinism(S):
    N, K = synth.C1_SHAPE
    say(f"f16 C1 S={S}")
    W, x = _case(N, K)
    y_ref, A = oracle.gemv_f16(W, x)
    Wd, xd = dev(W), dev(x)
    y1 = host(wsgemv.gemv_f16(Wd, xd, splits=S))
    y2 = host(wsgemv.gemv_f16(Wd, xd, splits=S))
    assert_within(y1, y_ref, A, f"S={S}")
    assert_bits_equal(y1, y2, "repeat run")


@pytest.mark.parametrize("N,K", [(1, 8), (1, 1024), (5, 16), (17, 1000), (63, 1032), (65, 3072),
                                 (100, 2056), (257, 512), (1000, 4096), (3, 16384), (2, 17000)])
def test_ragged_shapes(N, K):
    say(f"f16 ragged {N}x{K}")
    W, x = _case(N, K, workload=50, w_id=N, x_id=K)
    y_ref, A = oracle.gemv_f16(W, x)
    y = host(wsgemv.gemv_f16(dev(W), dev(x)))
    assert_within(y, y_ref, A, f"{N}x{K}")


@pytest.mark.parametrize("S", [2, 3, 5])
def test_ragged_split(S):
    N, K = 33, 1000 + 8 * S
    say(f"f16 ragged split {N}x{K} S={S}")
    W, x = _case(N, K, workload=51, w_id=S)
    y_ref, A = oracle.gemv_f16(W, x)
    y = host(wsgemv.gemv_f16(dev(W), dev(x), splits=S))
    assert_within(y, y_ref, A, f"S={S}")


def test_subnormal_weights_are_not_flushed():
    # Every weight is a subnormal fp16; flushing them to zero would give 0.
    N, K = 8, 1024
    say("f16 subnormals")
    bits = (np.arange(N * K, dtype=np.uint32) % 1023 + 1).astype(np.uint16).reshape(N, K)
    W = bits.view(np.float16)
    x = np.full(K, 1024.0, np.float16)
    y_ref, A = oracle.gemv_f16(W, x)
    assert np.all(y_ref > 0)
    y = host(wsgemv.gemv_f16(dev(W), dev(x)))
    assert_within(y, y_ref, A, "subnormal weights")


def test_power_of_two_scaling_is_exact():
    N, K = 300, 2048
    say("f16 scaling")
    W, x = _case(N, K, workload=52)
    Wd = dev(W)
    y1 = host(wsgemv.gemv_f16(Wd, dev(x)))
    y4 = host(wsgemv.gemv_f16(Wd, dev((x.astype(np.float32) * 4).astype(np.float16))))
    assert_bits_equal(y4, (4 * y1).astype(np.float32), "y(4x) == 4 y(x)")


def test_row_permutation_is_exact():
    N, K = 301, 1024
    say("f16 permutation")
    W, x = _case(N, K, workload=53)
    perm = np.random.default_rng(0).permutation(N)
    xd = dev(x)
    y = host(wsgemv.gemv_f16(dev(W), xd))
    yp = host(wsgemv.gemv_f16(dev(W[perm]), xd))
    assert_bits_equal(yp, y[perm], "permuted rows")


def test_identity_and_one_hot_exact():
    K = 512
    say("f16 identity")
    x = synth.f16_normal(54, 1, (K,), 1.0)
    y = host(wsgemv.gemv_f16(dev(np.eye(K, dtype=np.float16)), dev(x)))
    assert_bits_equal(y, x.astype(np.float32), "identity")


def test_degenerate_sizes():
    say("f16 N=0 / K=0")
    y = torch.full((4,), 7.0, device="cuda")
    wsgemv.gemv_f16(torch.empty((4, 0), dtype=torch.float16, device="cuda"),
                    torch.empty(0, dtype=torch.float16, device="cuda"), y=y)
    assert host(y).tolist() == [0.0] * 4            # empty sum
    y0 = torch.empty(0, device="cuda")
    wsgemv.gemv_f16(torch.empty((0, 64), dtype=torch.float16, device="cuda"),
                    torch.zeros(64, dtype=torch.float16, device="cuda"), y=y0)
    torch.cuda.synchronize()


@pytest.mark.parametrize("S", [0, 1, 2, 4])
def test_lm_head_248320x1024(S):
    N, K = synth.LMHEAD
    say(f"f16 lm_head {N}x{K} S={S}")
    W, x = _case(N, K, workload=2)
    y_ref, A = oracle.gemv_f16(W, x)
    Wd, xd = dev(W), dev(x)
    y = host(wsgemv.gemv_f16(Wd, xd, splits=S))
    assert_within(y, y_ref, A, f"lm_head S={S}")
    assert_bits_equal(host(wsgemv.gemv_f16(Wd, xd, splits=S)), y, "repeat")
