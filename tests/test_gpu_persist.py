"""The persistent dependency-respecting step (WSG_STEP_PERSISTENT): a list of
fp16 linears in which a linear reads (part of) an earlier linear's fp16
output, run as one cooperative launch per step.

The exact case uses signed permutation matrices scaled by powers of two:
every product, sum and rounding is exact, so every stage must equal the
oracle chain bit for bit, over several replays with new inputs; a stage that
read a stale or half-written input could not.  The random cases keep each
stage within the GEMV bound plus the propagated effect of the previous
stages' bounds and roundings, computed from the oracle's own chain.  The
give-up path is forced from the host (consumers wait for a tag no producer
writes, with a spin limit of a few polls): the launch still ends, the
give-ups are counted, and the next step is correct again."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_bits_equal, assert_within, dev, host, say
from weight_streaming_gemv_decode_amd import synth, wsgemv

pytestmark = pytest.mark.gpu


def _ulp16(v):
    v = np.maximum(np.abs(np.asarray(v, np.float64)), 2.0 ** -14)
    return 2.0 ** (np.floor(np.log2(v)) - 10)


def _chain(Ws, x0, prefix=True):
    """Linears on the GPU: stage i reads the leading K_i values of stage
    i-1's y16 (stage 0 reads x0)."""
    lins, ys, y16s = [], [], []
    x = dev(x0)
    for W in Ws:
        N, K = W.shape
        y = torch.empty(N, device="cuda")
        y16 = torch.empty(N, dtype=torch.float16, device="cuda")
        lins.append(wsgemv.Linear(wsgemv.F16, dev(W), x[:K], y, N, K, y16=y16))
        ys.append(y)
        y16s.append(y16)
        x = y16
    return lins, ys, y16s


def _signed_perm(r, K):
    W = np.zeros((K, K), np.float16)
    W[np.arange(K), r.permutation(K)] = r.choice([-1.0, 1.0], K) * 2.0 ** int(r.integers(-1, 2))
    return W


@pytest.mark.parametrize("K", [1024, 3072, 1000])
def test_exact_chain_bit_for_bit(K):
    say(f"persistent exact chain K={K}")
    r = synth.rng(180, K)
    depth = 8
    Ws = [_signed_perm(r, K) for _ in range(depth)]
    x_in = torch.empty(K, dtype=torch.float16, device="cuda")
    lins, ys, y16s = _chain(Ws, np.zeros(K, np.float16))
    lins[0] = wsgemv.Linear(wsgemv.F16, lins[0].W, x_in, ys[0], K, K, y16=y16s[0])
    step = wsgemv.DecodeStep(lins, wsgemv.STEP_PERSISTENT)
    launches, units = step.info()
    assert launches == 1 and units >= depth and not step.uses_graph()
    for rep in range(3):
        x0 = r.integers(-64, 65, K).astype(np.float16)
        x_in.copy_(torch.from_numpy(x0))
        for t in ys + y16s:
            t.fill_(float("nan"))
        step()
        want = oracle.chain_f16(Ws, x0)
        for i in range(depth):
            assert_bits_equal(host(ys[i]).astype(np.float64), want[i][0], f"stage {i} y, replay {rep}")
            assert_bits_equal(host(y16s[i]), want[i][1], f"stage {i} y16, replay {rep}")
    assert step.give_ups() == 0
    step.close()


def _check_propagated(Ws, x0, ys, y16s, what):
    """Every stage within its GEMV bound plus |W| times the previous stage's
    input bound; the kernel's y16 is its own y rounded to fp16."""
    x = np.asarray(x0, np.float16)
    tol_x = np.zeros(x.size)
    for i, W in enumerate(Ws):
        N, K = W.shape
        y_ref, A = oracle.gemv_f16(W, x[:K])
        # |W| @ tol in fp32 (non-negative terms: relative error below K * 2^-24, inside the 1.001)
        prop = (np.abs(W.astype(np.float32)) @ tol_x[:K].astype(np.float32)).astype(np.float64)
        tol = oracle.bound(A) + 1.001 * prop
        y = host(ys[i]).astype(np.float64)
        err = np.abs(y - y_ref)
        assert np.all(np.isfinite(y)) and np.all(err <= tol), \
            f"{what} stage {i}: max err / tol = {float(np.max(err / tol)):.3g}"
        assert_bits_equal(host(y16s[i]), host(ys[i]).astype(np.float16), f"{what} stage {i} y16")
        x = oracle.round_f16(y_ref)
        tol_x = tol + _ulp16(np.abs(y_ref) + tol)


def test_decode_layer_chain_within_propagated_bound():
    """Two decode layers of the decode-step shapes chained through prefixes of
    y16 (2048 -> 1024, 6144 -> 3072), then a 50000-row head; unit-gain
    weights keep the values in range; two replays with new inputs are
    bit-identical to each other when the input repeats."""
    say("persistent decode-layer chain")
    shapes = [(2048, 1024), (1024, 1024), (6144, 1024), (1024, 3072)] * 2 + [(50000, 1024)]
    Ws = [synth.f16_normal(181, i, (N, K), 1.0 / np.sqrt(K)) for i, (N, K) in enumerate(shapes)]
    x_in = torch.empty(1024, dtype=torch.float16, device="cuda")
    lins, ys, y16s = _chain(Ws, np.zeros(1024, np.float16))
    N0, K0 = shapes[0]
    lins[0] = wsgemv.Linear(wsgemv.F16, lins[0].W, x_in, ys[0], N0, K0, y16=y16s[0])
    step = wsgemv.DecodeStep(lins, wsgemv.STEP_PERSISTENT)
    first = None
    for rep in range(3):
        x0 = synth.f16_normal(182, rep % 2, (1024,), synth.X_SIGMA)
        x_in.copy_(torch.from_numpy(x0))
        step()
        _check_propagated(Ws, x0, ys, y16s, f"replay {rep}")
        _check_each_stage(Ws, x0, ys, y16s, f"replay {rep}")
        out = [host(y).copy() for y in ys]
        if rep == 0:
            first = out
        if rep == 2:
            for i in range(len(ys)):
                assert_bits_equal(out[i], first[i], f"stage {i}: same input, same bits")
    assert step.give_ups() == 0
    step.close()


def _check_each_stage(Ws, x0, ys, y16s, what):
    """Every stage against the oracle on the input that stage actually read
    (the GPU's previous fp16 output, or x0): within the GEMV bound, and y16
    its own y rounded.  A stage that read a stale or half-written input
    would have computed the product of a different vector."""
    x = np.asarray(x0, np.float16)
    for i, W in enumerate(Ws):
        N, K = W.shape
        y_ref, A = oracle.gemv_f16(W, x[:K])
        y = host(ys[i])
        assert_within(y, y_ref, A, f"{what} stage {i}")
        x = host(y16s[i])
        assert_bits_equal(x, y.astype(np.float16), f"{what} stage {i} y16")


def test_full_decode_step_chain():
    """The 113-linear decode step as one dependent chain, as the bench runs
    it (each linear reads the leading K values of the previous one's y16;
    the decode-step weights, ~N(0, 0.02)), replayed with a new first input
    each time: every stage within the GEMV bound of its own input."""
    say("persistent full decode-step chain")
    step_in = synth.decode_step_f16(workload=3)
    Ws = [W for _, W, _ in step_in]
    K0 = Ws[0].shape[1]
    x_in = torch.empty(K0, dtype=torch.float16, device="cuda")
    lins, ys, y16s = _chain(Ws, np.zeros(K0, np.float16))
    lins[0] = wsgemv.Linear(wsgemv.F16, lins[0].W, x_in, ys[0], Ws[0].shape[0], K0, y16=y16s[0])
    step = wsgemv.DecodeStep(lins, wsgemv.STEP_PERSISTENT)
    for rep in range(2):
        x0 = synth.f16_normal(185, rep, (K0,), synth.X_SIGMA) if rep else step_in[0][2]
        x_in.copy_(torch.from_numpy(x0))
        step()
        _check_each_stage(Ws, x0, ys, y16s, f"C3 chain replay {rep}")
    assert step.give_ups() == 0
    step.close()


def test_independent_and_mixed_inputs():
    """Linears with plain inputs beside chained ones, an input taken from the
    middle of an earlier y16, and a ragged K; all within the GEMV bound (the
    chained ones within the propagated bound of their single producer)."""
    say("persistent mixed inputs")
    W0 = synth.f16_normal(183, 0, (3000, 1024), 1.0 / 32)
    W1 = synth.f16_normal(183, 1, (777, 1000), 1.0 / 32)      # reads y16_0[1000:2000]
    W2 = synth.f16_normal(183, 2, (513, 2056), 0.02)          # plain input, ragged K
    W3 = synth.f16_normal(183, 3, (64, 1024), 1.0 / 32)       # reads y16_0[0:1024]
    x0 = synth.f16_normal(183, 4, (1024,), 1.0)
    x2 = synth.f16_normal(183, 5, (2056,), 1.0)
    y16_0 = torch.empty(3000, dtype=torch.float16, device="cuda")
    ys = [torch.empty(n, device="cuda") for n in (3000, 777, 513, 64)]
    y16s = [y16_0] + [torch.empty(n, dtype=torch.float16, device="cuda") for n in (777, 513, 64)]
    lins = [wsgemv.Linear(wsgemv.F16, dev(W0), dev(x0), ys[0], 3000, 1024, y16=y16_0),
            wsgemv.Linear(wsgemv.F16, dev(W1), y16_0[1000:2000], ys[1], 777, 1000, y16=y16s[1]),
            wsgemv.Linear(wsgemv.F16, dev(W2), dev(x2), ys[2], 513, 2056, y16=y16s[2]),
            wsgemv.Linear(wsgemv.F16, dev(W3), y16_0[:1024], ys[3], 64, 1024)]
    step = wsgemv.DecodeStep(lins, wsgemv.STEP_PERSISTENT)
    for _ in range(2):
        step()
    y0_ref, A0 = oracle.gemv_f16(W0, x0)
    assert_within(host(ys[0]), y0_ref, A0, "producer")
    assert_within(host(ys[2]), *oracle.gemv_f16(W2, x2), "plain ragged")
    x0r = oracle.round_f16(y0_ref)
    tol0 = oracle.bound(A0)
    tolx = tol0 + _ulp16(np.abs(y0_ref) + tol0)
    for W, sl, y, what in ((W1, slice(1000, 2000), ys[1], "middle of y16"), (W3, slice(0, 1024), ys[3], "prefix")):
        ref, A = oracle.gemv_f16(W, x0r[sl])
        tol = oracle.bound(A) + 1.001 * (np.abs(W.astype(np.float64)) @ tolx[sl])
        err = np.abs(host(y).astype(np.float64) - ref)
        assert np.all(err <= tol), f"{what}: max err / tol = {float(np.max(err / tol)):.3g}"
    assert step.give_ups() == 0
    step.close()


def test_give_up_path_ends_and_is_counted():
    """Consumers wait for a tag no producer writes, with a spin limit of 4
    polls: the launch ends, the give-ups are counted, and with the switch
    off the same plan computes the exact chain again."""
    say("persistent give-up path")
    K = 1024
    r = synth.rng(184, 0)
    Ws = [_signed_perm(r, K) for _ in range(4)]
    x0 = r.integers(-64, 65, K).astype(np.float16)
    lins, ys, y16s = _chain(Ws, x0)
    step = wsgemv.DecodeStep(lins, wsgemv.STEP_PERSISTENT)
    try:
        wsgemv.tune_set("chain_spin_limit", 4)
        wsgemv.tune_set("chain_test_stale", 1)
        step()
        torch.cuda.synchronize()
        n = step.give_ups()
        assert n >= 1, n
    finally:
        wsgemv.tune_set("chain_test_stale", -1)
        wsgemv.tune_set("chain_spin_limit", -1)
    assert step.give_ups() == 0                      # the count was cleared by the previous read
    step()
    want = oracle.chain_f16(Ws, x0)
    for i in range(len(Ws)):
        assert_bits_equal(host(y16s[i]), want[i][1], f"stage {i} after the forced give-ups")
    assert step.give_ups() == 0
    step.close()


def test_trace_records_every_unit_and_leaves_outputs_alone():
    """A traced step (wsg_decode_step_trace) writes, for every work unit in
    list order, start <= input staged <= finished on one clock, its linear
    (non-decreasing along the list, every linear present) and a workgroup
    inside the grid; its outputs equal the untraced step's bit for bit, and
    with tracing stopped the buffer is no longer written."""
    say("persistent trace")
    K = 1024
    r = synth.rng(185, 0)
    Ws = [_signed_perm(r, K) for _ in range(5)] + [synth.f16_normal(185, 1, (3000, K), 1.0 / np.sqrt(K))]
    x0 = r.integers(-64, 65, K).astype(np.float16)
    lins, ys, y16s = _chain(Ws, x0)
    step = wsgemv.DecodeStep(lins, wsgemv.STEP_PERSISTENT)
    step()
    plain = [host(y).copy() for y in ys]
    units = step.info()[1]
    with pytest.raises(wsgemv.WsgError):
        step.set_trace(torch.zeros(4 * units - 1, dtype=torch.int64, device="cuda"))   # too small
    buf = torch.zeros(4 * units, dtype=torch.int64, device="cuda")
    step.set_trace(buf)
    step()
    traced = [host(y).copy() for y in ys]
    for i in range(len(ys)):
        assert_bits_equal(traced[i], plain[i], f"stage {i}: traced step")
    t = host(buf).reshape(units, 4)
    lin = t[:, 3] & 0xFFFFFFFF
    wg = t[:, 3] >> 32
    assert np.all(t[:, 0] > 0) and np.all(t[:, 0] <= t[:, 1]) and np.all(t[:, 1] <= t[:, 2])
    assert np.all(np.diff(lin) >= 0) and set(lin.tolist()) == set(range(len(Ws)))
    assert np.all(wg >= 0) and np.all(wg < units)
    span_us = (t[:, 2].max() - t[:, 0].min()) * 0.01                      # 100 MHz clock
    assert 0.5 < span_us < 1e5, span_us
    step.set_trace(None)
    buf.zero_()
    step()
    torch.cuda.synchronize()
    assert int(buf.abs().sum().item()) == 0
    assert step.give_ups() == 0
    step.close()


@pytest.mark.parametrize("seed", range(4))
def test_random_chains(seed):
    """Seeded random chains: 3..7 stages, each reading K values (any multiple
    of 8 up to 4096) that start any multiple of 8 into the previous stage's
    y16, N up to 6000; two replays with new first inputs; every stage against
    the oracle on the input it actually read, y16 its own y rounded."""
    r = synth.rng(186, seed)
    depth = int(r.integers(3, 8))
    Ks, offs, Ns = [8 * int(r.integers(1, 513))], [0], []
    for i in range(depth):
        if i + 1 < depth:
            Kn = 8 * int(r.integers(1, 513))
            o = 8 * int(r.integers(0, 65))
            Ns.append(int(r.integers(o + Kn, max(o + Kn, 6000) + 1)))
            Ks.append(Kn)
            offs.append(o)
        else:
            Ns.append(int(r.integers(1, 6001)))
    say(f"persistent random chain seed={seed}: N={Ns} K={Ks} offsets={offs}")
    Ws = [synth.f16_normal(187, 16 * seed + i, (Ns[i], Ks[i]), 1.0 / np.sqrt(Ks[i])) for i in range(depth)]
    x_in = torch.empty(Ks[0], dtype=torch.float16, device="cuda")
    lins, ys, y16s = [], [], []
    x = x_in
    for i in range(depth):
        y = torch.empty(Ns[i], device="cuda")
        y16 = torch.empty(Ns[i], dtype=torch.float16, device="cuda")
        lins.append(wsgemv.Linear(wsgemv.F16, dev(Ws[i]), x, y, Ns[i], Ks[i], y16=y16))
        ys.append(y)
        y16s.append(y16)
        if i + 1 < depth:
            x = y16[offs[i + 1]:offs[i + 1] + Ks[i + 1]]
    step = wsgemv.DecodeStep(lins, wsgemv.STEP_PERSISTENT)
    for rep in range(2):
        x0 = synth.f16_normal(188, 2 * seed + rep, (Ks[0],), 1.0)
        x_in.copy_(torch.from_numpy(x0))
        step()
        xin = x0
        for i in range(depth):
            y_ref, A = oracle.gemv_f16(Ws[i], xin)
            y = host(ys[i])
            assert_within(y, y_ref, A, f"seed {seed} replay {rep} stage {i}")
            y16 = host(y16s[i])
            assert_bits_equal(y16, y.astype(np.float16), f"seed {seed} replay {rep} stage {i} y16")
            if i + 1 < depth:
                xin = y16[offs[i + 1]:offs[i + 1] + Ks[i + 1]]
    assert step.give_ups() == 0
    step.close()
