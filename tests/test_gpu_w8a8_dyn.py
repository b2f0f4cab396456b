"""int8 weights x fp16 activations quantised per token in the kernel
(gemv_w8a8_dyn, decode-step kind W8A8_DYN): the codes and the scale bit
for bit against the oracle's quantiser, the int32 accumulators bit for bit
against the oracle's W8A8 product on the oracle's own codes, and y within
the parity bound."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_bits_equal, assert_within, dev, host, say
from weight_streaming_gemv_decode_amd import synth, wsgemv

pytestmark = pytest.mark.gpu


def _case(N, K, workload=140, x_sigma=synth.X_SIGMA):
    Wq = synth.int8_uniform(workload, 0, (N, K))
    sw = synth.f32_uniform(workload, 1, (N,), 0.001, 0.01)
    x = synth.f16_normal(workload, 2, (K,), x_sigma)
    return Wq, sw, x


def _check(Wq, sw, x, splits=0, what="", dirty_ws=False):
    N, K = Wq.shape
    acc = torch.full((N,), -7, dtype=torch.int32, device="cuda")
    xq = torch.full((max(K, 1),), 99, dtype=torch.int8, device="cuda")
    sx = torch.full((1,), float("nan"), device="cuda")
    ws = wsgemv.workspace(wsgemv.W8A8_DYN, 1, N, K, splits)
    if dirty_ws and ws is not None:
        # NaN bits over the partials and the published scale (everything before
        # the arrival counters, which start at zero): both must be written before use
        S = splits or wsgemv.plan_splits(wsgemv.W8A8_DYN, 1, N, K)
        ws[:(S * N * 4 + 256 + 255) // 256 * 256].fill_(0xFF)
    y = wsgemv.gemv_w8a8_dyn(dev(Wq), dev(sw), dev(x), acc_out=acc, xq_out=xq[:K] if K else None, sx_out=sx,
                             splits=splits, ws=ws)
    xq_ref, sx_ref = oracle.quantize_x_i8(x)
    assert_bits_equal(host(sx), np.array([sx_ref], np.float32), f"{what} scale")
    if K:
        assert_bits_equal(host(xq)[:K], xq_ref, f"{what} codes")
    acc_ref, y_ref, A = oracle.gemv_w8a8(Wq, sw, xq_ref, sx_ref)
    assert_bits_equal(host(acc), acc_ref, f"{what} accumulators")
    assert_within(host(y), y_ref, A, what)


# 8208..16384-wide rows (513..1024 code vectors) take the kernel that loads
# the row ahead of the weights; the others the late order
@pytest.mark.parametrize("N,K", [(1, 16), (17, 256), (100, 640), (1000, 2064), (14336, 4096), (4096, 14336),
                                 (77, 8208), (300, 16384), (5, 9216)])
def test_shapes(N, K):
    say(f"w8a8 dyn {N}x{K}")
    _check(*_case(N, K), what=f"{N}x{K}")


@pytest.mark.parametrize("S", [1, 2, 7])
@pytest.mark.parametrize("dirty", [False, True])
def test_splits(S, dirty):
    """k split across workgroups: every slice quantises its own codes with
    the same scale, which the first work unit also publishes in the
    workspace (partials and scale slots full of NaN bits change nothing)."""
    say(f"w8a8 dyn splits={S} dirty={dirty}")
    _check(*_case(300, 7168, workload=141), splits=S, what=f"S={S}", dirty_ws=dirty)
    # a row the early-order kernel holds, cut into S slices
    _check(*_case(130, 12288, workload=142), splits=S, what=f"12288 S={S}", dirty_ws=dirty)


def test_ties_to_even_and_clamp():
    """max|x| = 127 makes s_x = 1 exactly, so the codes are rint(x): the
    halves go to even, and nothing exceeds 127."""
    say("w8a8 dyn ties")
    K = 32
    x = np.zeros(K, np.float16)
    x[:10] = [127, -127, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, 126.5, -0.5]
    Wq = synth.int8_uniform(142, 0, (8, K))
    sw = np.full(8, 0.5, np.float32)
    _check(Wq, sw, x, what="ties")
    xq, sx = oracle.quantize_x_i8(x)
    assert sx == np.float32(1.0) and xq[:10].tolist() == [127, -127, 2, 4, -2, -4, 0, 2, 126, 0]


def test_zero_and_tiny_activations():
    say("w8a8 dyn zero/tiny")
    Wq, sw, _ = _case(64, 512, workload=143)
    _check(Wq, sw, np.zeros(512, np.float16), what="all zero")
    x = np.zeros(512, np.float16)
    x[::7] = np.float16(6e-8)                      # subnormal fp16 activations
    _check(Wq, sw, x, what="subnormal")
    x = np.full(512, -np.float16(60000.0), np.float16)
    _check(Wq, sw, x, what="large negative")


def test_k_zero():
    say("w8a8 dyn K=0")
    N = 40
    y = torch.full((N,), 3.0, device="cuda")
    acc = torch.full((N,), 5, dtype=torch.int32, device="cuda")
    sx = torch.full((1,), float("nan"), device="cuda")
    wsgemv.gemv_w8a8_dyn(torch.empty((N, 0), dtype=torch.int8, device="cuda"), torch.ones(N, device="cuda"),
                         torch.empty(0, dtype=torch.float16, device="cuda"), y=y, acc_out=acc, sx_out=sx)
    assert np.all(host(y) == 0) and np.all(host(acc) == 0) and host(sx)[0] == 0


@pytest.mark.parametrize("mode", [wsgemv.STEP_GROUPED, wsgemv.STEP_ORDERED, wsgemv.STEP_ORDERED | wsgemv.STEP_FORCE_GRAPH])
def test_in_decode_steps(mode):
    """W8A8_DYN linears beside an fp16 one, one of them taking the greedy
    token, one split over k (ORDERED); two replays with new activations."""
    say(f"w8a8 dyn step mode={mode:#x}")
    r = synth.rng(144, 0)
    specs = [(2048, 1024), (1024, 3072), (300, 1024)]
    lins, cases = [], []
    tok = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    for i, (N, K) in enumerate(specs):
        Wq, sw, _ = _case(N, K, workload=145 + i)
        xb = torch.empty(K, dtype=torch.float16, device="cuda")
        y = torch.empty(N, device="cuda")
        acc = torch.empty(N, dtype=torch.int32, device="cuda")
        kw = {"argmax_idx": tok} if i == 0 else {}
        splits = 2 if (i == 1 and not mode & wsgemv.STEP_GROUPED) else 0
        lins.append(wsgemv.Linear(wsgemv.W8A8_DYN, dev(Wq), xb, y, N, K, scale=dev(sw), acc_out=acc,
                                  splits=splits, **kw))
        cases.append((Wq, sw, xb, y, acc))
    Wf = synth.f16_normal(148, 0, (500, 1024), synth.W_SIGMA)
    xf = synth.f16_normal(148, 1, (1024,), synth.X_SIGMA)
    yf = torch.empty(500, device="cuda")
    lins.append(wsgemv.Linear(wsgemv.F16, dev(Wf), dev(xf), yf, 500, 1024))
    step = wsgemv.DecodeStep(lins, mode)
    for rep in range(2):
        xs = []
        for i, (Wq, sw, xb, y, acc) in enumerate(cases):
            x = r.normal(0, 1 + rep, xb.numel()).astype(np.float16)
            xb.copy_(dev(x))
            xs.append(x)
        step()
        for i, ((Wq, sw, xb, y, acc), x) in enumerate(zip(cases, xs)):
            xq_ref, sx_ref = oracle.quantize_x_i8(x)
            acc_ref, y_ref, A = oracle.gemv_w8a8(Wq, sw, xq_ref, sx_ref)
            assert_bits_equal(host(acc), acc_ref, f"linear {i} accumulators, replay {rep}")
            assert_within(host(y), y_ref, A, f"linear {i}, replay {rep}")
            if i == 0:
                t = int(host(tok)[0])
                assert t == oracle.argmax_f32(host(y)) and oracle.argmax_is_valid(t, y_ref, A), t
    yf_ref, Af = oracle.gemv_f16(Wf, xf)
    assert_within(host(yf), yf_ref, Af, "fp16 linear")
    step.close()


def test_fed_by_an_fp16_linear():
    """A dependent pair in an ORDERED plan: an fp16 signed permutation (its
    y16 equals the oracle's exactly) feeds a W8A8_DYN linear."""
    say("w8a8 dyn fed through y16")
    K, N = 1024, 777
    r = synth.rng(149, 0)
    x0 = r.integers(-64, 65, K).astype(np.float16)
    P = np.zeros((K, K), np.float16)
    P[np.arange(K), r.permutation(K)] = r.choice([-1.0, 1.0], K) * 0.5
    Wq, sw, _ = _case(N, K, workload=150)
    y16 = torch.empty(K, dtype=torch.float16, device="cuda")
    acc = torch.empty(N, dtype=torch.int32, device="cuda")
    y = torch.empty(N, device="cuda")
    lins = [wsgemv.Linear(wsgemv.F16, dev(P), dev(x0), torch.empty(K, device="cuda"), K, K, y16=y16),
            wsgemv.Linear(wsgemv.W8A8_DYN, dev(Wq), y16, y, N, K, scale=dev(sw), acc_out=acc)]
    step = wsgemv.DecodeStep(lins, wsgemv.STEP_ORDERED)
    step()
    x1 = oracle.round_f16(oracle.gemv_f16(P, x0)[0])
    assert_bits_equal(host(y16), x1, "fp16 stage y16")
    xq_ref, sx_ref = oracle.quantize_x_i8(x1)
    acc_ref, y_ref, A = oracle.gemv_w8a8(Wq, sw, xq_ref, sx_ref)
    assert_bits_equal(host(acc), acc_ref, "W8A8_DYN accumulators")
    assert_within(host(y), y_ref, A, "W8A8_DYN y")
    step.close()
