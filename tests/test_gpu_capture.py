"""The library's launches captured by the caller into a graph of their own
(torch.cuda.graph): an EAGER decode step mixing fp16 (split over k, taking
the greedy token), W8A8 with in-kernel quantisation, int4 with the
causal-conv1d step, and two standalone calls (top-k, split fp16 GEMV).
The graph is replayed three times with new activations written between the
replays, with eager work and synchronisations in between, and every replay
is checked against the oracle.  Nothing the library launches may be a
memset node; zeroing is done by kernels."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_bits_equal, assert_within, dev, host, say
from weight_streaming_gemv_decode_amd import synth, wsgemv

pytestmark = pytest.mark.gpu


def test_caller_captured_graph_replays():
    say("caller-captured graph")
    r = synth.rng(180, 0)
    # an fp16 linear split over k, taking the greedy token
    N1, K1 = 3000, 2048
    W1 = synth.f16_normal(180, 1, (N1, K1), synth.W_SIGMA)
    x1 = torch.empty(K1, dtype=torch.float16, device="cuda")
    y1 = torch.empty(N1, device="cuda")
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    # W8A8 with fp16 activations quantised in the kernel
    N2, K2 = 1024, 1024
    Wq = synth.int8_uniform(180, 2, (N2, K2))
    sw = synth.f32_uniform(180, 3, (N2,), 0.001, 0.01)
    x2 = torch.empty(K2, dtype=torch.float16, device="cuda")
    y2 = torch.empty(N2, device="cuda")
    acc2 = torch.empty(N2, dtype=torch.int32, device="cuda")
    # int4 with the conv step over its output
    N3, K3, W = 512, 1024, 4
    Wc = synth.w4_words(180, 4, N3, K3)
    s4 = synth.f16_uniform(180, 5, (N3, K3 // 128), 0.002, 0.02)
    Wp, Sp = wsgemv.pack_w4(dev(Wc), dev(s4))
    x3 = torch.empty(K3, dtype=torch.float16, device="cuda")
    y3 = torch.empty(N3, device="cuda")
    cw = r.normal(0, 0.5, (N3, W)).astype(np.float16)
    cb = r.normal(0, 1, N3).astype(np.float32)
    st0 = r.normal(0, 1, (N3, W - 1)).astype(np.float32)
    cst = dev(st0)
    cout = torch.empty(N3, device="cuda")
    lins = [wsgemv.Linear(wsgemv.F16, dev(W1), x1, y1, N1, K1, splits=2, argmax_idx=tok),
            wsgemv.Linear(wsgemv.W8A8_DYN, dev(Wq), x2, y2, N2, K2, scale=dev(sw), acc_out=acc2),
            wsgemv.Linear(wsgemv.W4A16, Wp, x3, y3, N3, K3, scale=Sp, group=128, conv_w=dev(cw),
                          conv_bias=dev(cb), conv_state=cst, conv_out=cout, conv_silu=True)]
    stream = torch.cuda.Stream()
    step = wsgemv.DecodeStep(lins, wsgemv.STEP_ORDERED | wsgemv.STEP_EAGER, stream=stream)
    # standalone calls with their buffers made before capture
    k = 8
    tk_idx = torch.empty(k, dtype=torch.int32, device="cuda")
    tk_val = torch.empty(k, device="cuda")
    tk_ws = torch.zeros(wsgemv.lib().wsg_topk_ws_bytes(N1, k), dtype=torch.uint8, device="cuda")
    W5 = synth.f16_normal(180, 6, (700, 4096), synth.W_SIGMA)
    y5 = torch.empty(700, device="cuda")
    ws5 = wsgemv.workspace(wsgemv.F16, 1, 700, 4096, 3, "cuda")
    x5 = torch.empty(4096, dtype=torch.float16, device="cuda")

    def body():
        step(stream)
        wsgemv.topk_f32(y1, k, idx=tk_idx, val=tk_val, ws=tk_ws, stream=stream)
        wsgemv.gemv_f16(dev_W5, x5, y=y5, splits=3, ws=ws5, stream=stream)

    dev_W5 = dev(W5)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        body()                                    # warm-up outside the capture
    stream.synchronize()
    with torch.cuda.graph(g, stream=stream):
        body()
    cst.copy_(dev(st0))                           # the warm-up step advanced the conv state
    st_ref = st0.copy()
    for rep in range(3):
        xs = [synth.f16_normal(181, 10 * rep + i, (K,), synth.X_SIGMA) for i, K in enumerate((K1, K2, K3, 4096))]
        for buf, x in zip((x1, x2, x3, x5), xs):
            buf.copy_(dev(x))
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").sum()   # the program's own eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        y1_ref, A1 = oracle.gemv_f16(W1, xs[0])
        assert_within(host(y1), y1_ref, A1, f"fp16 split, replay {rep}")
        t = int(host(tok)[0])
        assert t == oracle.argmax_f32(host(y1)) and oracle.argmax_is_valid(t, y1_ref, A1), (rep, t)
        assert np.array_equal(host(tk_idx).astype(np.int64), oracle.topk_f32(host(y1), k)), f"top-k, replay {rep}"
        xq, sx = oracle.quantize_x_i8(xs[1])
        acc_ref, y2_ref, A2 = oracle.gemv_w8a8(Wq, sw, xq, sx)
        assert_bits_equal(host(acc2), acc_ref, f"W8A8_DYN accumulators, replay {rep}")
        assert_within(host(y2), y2_ref, A2, f"W8A8_DYN, replay {rep}")
        y3_ref, A3 = oracle.gemv_w4a16(Wc, s4, xs[2])
        y3_ref, A3 = y3_ref.reshape(-1), A3.reshape(-1)
        assert_within(host(y3), y3_ref, A3, f"int4, replay {rep}")
        # the conv ran on the kernel's own y3: its state's newest tap is y3 bit for bit
        assert_bits_equal(host(cst)[:, W - 2], host(y3), f"conv state, replay {rep}")
        want, A_c, st_ref = oracle.causal_conv1d_step(y3_ref.astype(np.float32), cw, cb, st_ref, True)
        taps = np.abs(cw.astype(np.float64))
        bnd = oracle.conv_bound(A_c, want, True) + 1.1 * taps[:, W - 1] * oracle.bound(A3)
        if rep == 0:   # later replays carry earlier steps' GEMV bounds in the state; the first is exact
            err = np.abs(host(cout).astype(np.float64) - want)
            assert np.all(err <= bnd), f"conv out, replay {rep}"
        y5_ref, A5 = oracle.gemv_f16(W5, xs[3])
        assert_within(host(y5), y5_ref, A5, f"standalone split GEMV, replay {rep}")
    step.close()
