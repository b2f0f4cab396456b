"""Causal-conv1d decode step on the GPU: the standalone step over a given
input, and the step fused into the epilogue of the linear whose output it
convolves.  Outputs against the oracle within the conv bound, and the
updated state bit for bit (it holds copies of fp32 inputs)."""
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


def _within(got, want, bnd, what):
    err = np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))
    r = float(np.max(err / bnd)) if err.size else 0.0
    assert np.all(np.isfinite(got)) and r <= 1.0, f"{what}: max err / bound = {r:.3g}"


def test_golden():
    say("conv1d golden")
    g = json.load(open(os.path.join(GOLDEN, "conv1d_step.json")))
    for c in g["cases"]:
        w = torch.tensor(np.array(c["w"], np.float16), device="cuda")
        st = torch.tensor(np.array(c["state"], np.float32), device="cuda")
        b = None if c["bias"] is None else torch.tensor(np.array(c["bias"], np.float32), device="cuda")
        out = wsgemv.causal_conv1d_step(torch.tensor(np.array(c["x"], np.float32), device="cuda"), w, st, bias=b,
                                        silu=c["silu"])
        _within(host(out), c["out"], 1e-6 * (1 + np.abs(c["out"])), "golden")
        assert host(st).tolist() == c["new_state"]


@pytest.mark.parametrize("C", [1, 7, 2048, 4099])
@pytest.mark.parametrize("W", [2, 3, 4, 8])
@pytest.mark.parametrize("silu,use_bias", [(False, False), (True, True)])
def test_steps_against_oracle(C, W, silu, use_bias):
    say(f"conv1d C={C} W={W} silu={silu} bias={use_bias}")
    r = synth.rng(130, C * 16 + W)
    w = r.normal(0, 0.5, (C, W)).astype(np.float16)
    b = r.normal(0, 1, C).astype(np.float32) if use_bias else None
    st_ref = r.normal(0, 1, (C, W - 1)).astype(np.float32)
    st = dev(st_ref)
    wd, bd = dev(w), (dev(b) if use_bias else None)
    for t in range(W + 2):                      # long enough for the whole window to turn over
        x = r.normal(0, 2, C).astype(np.float32)
        out = wsgemv.causal_conv1d_step(dev(x), wd, st, bias=bd, silu=silu)
        want, A, st_ref = oracle.causal_conv1d_step(x, w, b, st_ref, silu)
        _within(host(out), want, oracle.conv_bound(A, want, silu), f"step {t}")
        assert_bits_equal(host(st), st_ref, f"state after step {t}")


def test_zero_channels_is_a_no_op():
    say("conv1d C=0")
    w = torch.empty((0, 4), dtype=torch.float16, device="cuda")
    st = torch.empty((0, 3), device="cuda")
    out = wsgemv.causal_conv1d_step(torch.empty(0, device="cuda"), w, st)
    assert out.numel() == 0


def _fused_case(kind, N, K, W, silu, workload):
    r = synth.rng(workload, 0)
    cw = r.normal(0, 0.5, (N, W)).astype(np.float16)
    cb = r.normal(0, 1, N).astype(np.float32)
    st0 = r.normal(0, 1, (N, W - 1)).astype(np.float32)
    return cw, cb, st0


@pytest.mark.parametrize("mode", [wsgemv.STEP_ORDERED, wsgemv.STEP_ORDERED | wsgemv.STEP_FORCE_GRAPH, wsgemv.STEP_GROUPED,
                                  wsgemv.STEP_GROUPED | wsgemv.STEP_FORCE_GRAPH, wsgemv.STEP_GROUPED | wsgemv.STEP_EAGER])
@pytest.mark.parametrize("silu", [False, True])
def test_fused_into_f16_linear(mode, silu):
    """The conv step over a 2048 x 1024 linear's output inside its kernel;
    three replays with new activations.  The oracle runs the same chain on
    its own exact outputs; the bound adds, per tap, the GEMV bound of the
    output that tap saw."""
    say(f"conv1d fused f16 mode={mode:#x} silu={silu}")
    N, K, W = 2048, 1024, 4
    Wm = synth.f16_normal(131, 0, (N, K), synth.W_SIGMA)
    cw, cb, st0 = _fused_case(wsgemv.F16, N, K, W, silu, 132)
    x_buf = torch.empty(K, dtype=torch.float16, device="cuda")
    y = torch.empty(N, device="cuda")
    out = torch.empty(N, device="cuda")
    st = dev(st0)
    lin = wsgemv.Linear(wsgemv.F16, dev(Wm), x_buf, y, N, K, conv_w=dev(cw), conv_bias=dev(cb), conv_state=st,
                        conv_out=out, conv_silu=silu)
    # an unrelated linear in the same plan
    W2 = synth.f16_normal(131, 1, (300, 1024), synth.W_SIGMA)
    x2 = synth.f16_normal(131, 2, (1024,), synth.X_SIGMA)
    y2 = torch.empty(300, device="cuda")
    step = wsgemv.DecodeStep([lin, wsgemv.Linear(wsgemv.F16, dev(W2), dev(x2), y2, 300, 1024)], mode)
    st_ref = st0.copy()
    gb_hist = [np.zeros(N)] * (W - 1)           # the initial state is exact on both sides
    ys = []
    for t in range(3):
        x = synth.f16_normal(133, t, (K,), synth.X_SIGMA)
        x_buf.copy_(dev(x))
        step()
        y_ref, A_y = oracle.gemv_f16(Wm, x)
        yh = host(y)
        assert_within(yh, y_ref, A_y, f"y step {t}")
        ys.append(yh.copy())
        want, A_c, st_ref = oracle.causal_conv1d_step(y_ref.astype(np.float32), cw, cb, st_ref, silu)
        # window tap j < W-1 holds an output from an earlier step (its GEMV
        # bound), tap W-1 this step's output
        taps = np.abs(cw.astype(np.float64))
        prop = sum(taps[:, j] * gb_hist[j] for j in range(W - 1)) + taps[:, W - 1] * oracle.bound(A_y)
        gb_hist = gb_hist[1:] + [oracle.bound(A_y)]
        bnd = oracle.conv_bound(A_c, want, silu) + (1.1 if silu else 1.0) * prop
        _within(host(out), want, bnd, f"conv step {t}")
        # the state now holds the kernel's own last outputs
        st_h = host(st)
        for j in range(W - 1):
            src = t - (W - 2) + j
            if src >= 0:
                assert_bits_equal(st_h[:, j], ys[src], f"state tap {j} after step {t}")
    y2_ref, A2 = oracle.gemv_f16(W2, x2)
    assert_within(host(y2), y2_ref, A2, "unrelated linear")
    step.close()


def test_fused_into_w8a8_split_and_zero_k():
    say("conv1d fused w8a8 split + K=0")
    N, K, W = 1000, 2048, 3
    Wq = synth.int8_uniform(134, 0, (N, K))
    xq = synth.int8_uniform(134, 1, (K,))
    sw = synth.f32_uniform(134, 2, (N,), 0.001, 0.01)
    xs = torch.tensor([synth.X_SCALE_W8A8], device="cuda")
    cw, cb, st0 = _fused_case(wsgemv.W8A8, N, K, W, True, 135)
    y = torch.empty(N, device="cuda")
    out = torch.empty(N, device="cuda")
    st = dev(st0)
    yz = torch.empty(64, device="cuda")
    outz = torch.empty(64, device="cuda")
    stz = dev(st0[:64])
    # splits=2: the conv step runs in the k-split reduce kernel
    lins = [wsgemv.Linear(wsgemv.W8A8, dev(Wq), dev(xq), y, N, K, scale=dev(sw), x_scale=xs, splits=2,
                          conv_w=dev(cw), conv_bias=dev(cb), conv_state=st, conv_out=out, conv_silu=True),
            wsgemv.Linear(wsgemv.F16, torch.empty((64, 0), dtype=torch.float16, device="cuda"),
                          torch.empty(0, dtype=torch.float16, device="cuda"), yz, 64, 0, conv_w=dev(cw[:64]),
                          conv_bias=dev(cb[:64]), conv_state=stz, conv_out=outz)]
    step = wsgemv.DecodeStep(lins, wsgemv.STEP_ORDERED | wsgemv.STEP_FORCE_GRAPH)
    step()
    acc, y_ref, A_y = oracle.gemv_w8a8(Wq, sw, xq, synth.X_SCALE_W8A8)
    assert_within(host(y), y_ref, A_y, "w8a8 y")
    want, A_c, st_ref = oracle.causal_conv1d_step(y_ref.astype(np.float32), cw, cb, st0, True)
    bnd = oracle.conv_bound(A_c, want, True) + 1.1 * np.abs(cw[:, W - 1].astype(np.float64)) * oracle.bound(A_y)
    _within(host(out), want, bnd, "w8a8 conv")
    # K = 0: y = 0, the conv sees x = 0
    want_z, A_z, st_z = oracle.causal_conv1d_step(np.zeros(64, np.float32), cw[:64], cb[:64], st0[:64], False)
    _within(host(outz), want_z, oracle.conv_bound(A_z, want_z, False), "K=0 conv")
    assert_bits_equal(host(stz), st_z, "K=0 state")
    step.close()


@pytest.mark.parametrize("kind,N,mode,splits", [
    (wsgemv.W4A16, 2048, wsgemv.STEP_GROUPED, 0),
    (wsgemv.W4A16, 1000, wsgemv.STEP_GROUPED | wsgemv.STEP_FORCE_GRAPH, 0),
    (wsgemv.W4A16, 1000, wsgemv.STEP_ORDERED, 2),             # the conv runs in the k-split reduce
    (wsgemv.W4A8, 1000, wsgemv.STEP_GROUPED, 0),
    (wsgemv.W4A8, 2048, wsgemv.STEP_ORDERED | wsgemv.STEP_FORCE_GRAPH, 2),
], ids=["w4a16-grouped", "w4a16-grouped-graph-ragged", "w4a16-ordered-split2", "w4a8-grouped-ragged",
        "w4a8-ordered-split2"])
def test_fused_into_int4_linear(kind, N, mode, splits):
    """The conv step over an int4 linear's output (M = 1), in the work
    unit's epilogue or in the k-split reduce; two replays with new
    activations.  Bound as for the fp16 case: the conv rule plus, per tap,
    the GEMV bound of the output that tap saw."""
    say(f"conv1d fused int4 kind={kind} N={N} mode={mode:#x} splits={splits}")
    K, W, silu = 1024, 4, True
    Wc = synth.w4_words(136, 0, N, K)
    s4 = synth.f16_uniform(136, 1, (N, K // 128), 0.002, 0.02)
    Wp, Sp = wsgemv.pack_w4(dev(Wc.view(np.int32)), dev(s4))
    cw, cb, st0 = _fused_case(kind, N, K, W, silu, 137)
    x_buf = torch.empty(K, dtype=torch.float16, device="cuda")
    y = torch.empty(N, device="cuda")
    out = torch.empty(N, device="cuda")
    st = dev(st0)
    lin = wsgemv.Linear(kind, Wp, x_buf, y, N, K, scale=Sp, group=128, splits=splits, conv_w=dev(cw),
                        conv_bias=dev(cb), conv_state=st, conv_out=out, conv_silu=silu)
    step = wsgemv.DecodeStep([lin], mode)
    st_ref = st0.copy()
    taps = np.abs(cw.astype(np.float64))
    gb_hist = [np.zeros(N)] * (W - 1)
    for t in range(2):
        x = synth.f16_normal(138, t, (K,), synth.X_SIGMA)
        x_buf.copy_(dev(x))
        step()
        if kind == wsgemv.W4A16:
            y_ref, A_y = oracle.gemv_w4a16(Wc, s4, x)
        else:
            xq, sx = oracle.quantize_x_i8(x)
            y_ref, A_y = oracle.gemv_w4a8(Wc, s4, xq, sx)
        y_ref, A_y = y_ref.reshape(N), A_y.reshape(N)
        assert_within(host(y), y_ref, A_y, f"y step {t}")
        want, A_c, st_ref = oracle.causal_conv1d_step(y_ref.astype(np.float32), cw, cb, st_ref, silu)
        prop = sum(taps[:, j] * gb_hist[j] for j in range(W - 1)) + taps[:, W - 1] * oracle.bound(A_y)
        gb_hist = gb_hist[1:] + [oracle.bound(A_y)]
        _within(host(out), want, oracle.conv_bound(A_c, want, silu) + 1.1 * prop, f"conv step {t}")
        # the newest state tap holds the kernel's own output of this step
        assert_bits_equal(host(st)[:, W - 2], host(y), f"state tap {W - 2} after step {t}")
    step.close()
