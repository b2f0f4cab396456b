"""Greedy token on the GPU: the standalone reduce over a given vector, the
lm_head GEMV with the token fused into the kernel that writes the logits,
and a decode step whose lm_head takes the token.

The token is an integer decided by floating point, so the decision is
checked in the kernel's own precision: it must equal the oracle's argmax
rule applied to the logits the kernel wrote (bit for bit), and those
logits must be within the parity bound of the oracle's exact product, with
the token a largest exact logit within that bound."""
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


def _token(y_dev, ws=None):
    tok = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    val = torch.full((1,), 12345.0, device="cuda")
    wsgemv.argmax_f32(y_dev, token=tok, token_logit=val, ws=ws)
    return int(host(tok)[0]), host(val)


def test_golden_cases():
    say("argmax golden")
    g = json.load(open(os.path.join(GOLDEN, "argmax_ties.json")))
    for c in g["cases"]:
        y = np.array([int(v, 16) for v in c["bits"]], np.uint32).view(np.float32)
        t, v = _token(dev(y))
        assert t == c["argmax"], c["note"]
        want = y[t:t + 1].copy()
        if want[0] == 0:
            want[0] = 0.0                       # the token's logit comes back as +0
        if np.isnan(want[0]):
            assert np.isnan(v[0]), c["note"]
        else:
            assert_bits_equal(v, want, c["note"])


@pytest.mark.parametrize("N", [1, 2, 255, 4096, 4097, 65537, 248320, (1 << 20) + 3])
def test_random_with_planted_ties(N):
    say(f"argmax random N={N}")
    r = synth.rng(120, N)
    y = np.round(r.normal(0, 40, N)).astype(np.float32)     # integers: many exact ties
    if N > 10:
        top = y.max() + 1
        for i in sorted(r.choice(N, 3, replace=False)):
            y[i] = top                          # three equal maxima
    t, v = _token(dev(y))
    assert t == oracle.argmax_f32(y)
    assert v[0] == y[t]


def test_nan_inf_and_signed_zero_vectors():
    say("argmax nan/inf/zero")
    N = 100000
    y = np.full(N, np.nan, np.float32)
    assert _token(dev(y))[0] == 0                           # all NaN
    y[77777] = -np.inf
    assert _token(dev(y))[0] == 77777                       # -inf beats NaN
    y = np.full(N, -0.0, np.float32)
    y[5000] = 0.0
    assert _token(dev(y))[0] == 0                           # -0 equals +0
    y = np.full(N, -1.0, np.float32)
    y[60000] = np.inf
    y[90000] = np.inf
    y[::7] = np.nan
    assert _token(dev(y))[0] == oracle.argmax_f32(y) == 60000


def test_workspace_contents_do_not_matter_and_calls_repeat():
    say("argmax ws garbage + repeats")
    ws = torch.full((wsgemv.ARGMAX_WS_BYTES,), 0xFF, dtype=torch.uint8, device="cuda")
    r = synth.rng(121, 0)
    for rep in range(6):
        y = r.normal(0, 1, 300000).astype(np.float32)
        assert _token(dev(y), ws=ws)[0] == oracle.argmax_f32(y), rep


def _lm_case(N, K, workload=122):
    W = synth.f16_normal(workload, 0, (N, K), synth.W_SIGMA)
    x = synth.f16_normal(workload, 1, (K,), synth.X_SIGMA)
    return W, x


def _check_fused(W, x, y, tok, val, what):
    y_ref, A = oracle.gemv_f16(W, x)
    assert_within(y, y_ref, A, what)
    assert tok == oracle.argmax_f32(y), f"{what}: token is not the argmax of the kernel's own logits"
    assert oracle.argmax_is_valid(tok, y_ref, A), f"{what}: token is not a largest exact logit"
    assert val[0] == y[tok]


@pytest.mark.parametrize("S", [0, 1, 2, 3])
def test_lm_head_full_fused(S):
    """The full 248320 x 1024 lm_head with the token fused (S > 1: in the reduce)."""
    say(f"argmax lm_head S={S}")
    W, x = _lm_case(*synth.LMHEAD)
    Wd, xd = dev(W), dev(x)
    tokd = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    vald = torch.empty(1, device="cuda")
    y, _ = wsgemv.gemv_f16_argmax(Wd, xd, token=tokd, token_logit=vald, splits=S)
    _check_fused(W, x, host(y), int(host(tokd)[0]), host(vald), f"S={S}")
    # same logits as the plain GEMV
    assert_bits_equal(host(y), host(wsgemv.gemv_f16(Wd, xd, splits=S)), "fused vs plain logits")


def test_planted_maximum_and_tie():
    """A row with a margin far beyond the bound is the token; a bit-identical
    copy of it at a lower index takes the token (ties to the lowest index)."""
    say("argmax planted max + tie")
    N, K = 50000, 1024
    W, x = _lm_case(N, K, workload=123)
    xs = x.astype(np.float32)
    W[31337] = np.clip(np.sign(xs) * 0.5, -1, 1).astype(np.float16)   # aligned with x: logit ~ 0.4 K
    Wd, xd = dev(W), dev(x)
    y, tok = wsgemv.gemv_f16_argmax(Wd, xd)
    y_ref, A = oracle.gemv_f16(W, x)
    assert int(host(tok)[0]) == 31337 == int(np.argmax(y_ref))
    W[1234] = W[31337]
    W[40000] = W[31337]
    y, tok = wsgemv.gemv_f16_argmax(dev(W), xd)
    assert int(host(tok)[0]) == 1234
    _check_fused(W, x, host(y), 1234, host(y)[1234:1235], "tie")


@pytest.mark.parametrize("N,K", [(1, 8), (7, 64), (300, 1000), (4096, 4096), (17, 16384)])
def test_small_shapes_fused(N, K):
    say(f"argmax gemv {N}x{K}")
    W, x = _lm_case(N, K, workload=124 + N)
    y, tok = wsgemv.gemv_f16_argmax(dev(W), dev(x))
    yh = host(y)
    _check_fused(W, x, yh, int(host(tok)[0]), yh[int(host(tok)[0]):][:1], f"{N}x{K}")


def test_k_zero_gives_token_zero():
    say("argmax K=0")
    W = torch.empty((5, 0), dtype=torch.float16, device="cuda")
    x = torch.empty((0,), dtype=torch.float16, device="cuda")
    val = torch.full((1,), 9.0, device="cuda")
    y, tok = wsgemv.gemv_f16_argmax(W, x, token_logit=val)
    assert int(host(tok)[0]) == 0 and host(val)[0] == 0 and not host(y).any()


def _step_lins(step_in, tok, val):
    lins, refs = [], []
    for name, W, x in step_in:
        N, K = W.shape
        y = torch.full((N,), float("nan"), device="cuda")
        kw = dict(argmax_idx=tok, argmax_val=val) if name == "lm_head" else {}
        lins.append(wsgemv.Linear(wsgemv.F16, dev(W), dev(x), y, N, K, **kw))
        refs.append((W, x))
    return lins, refs


@pytest.mark.parametrize("mode", [wsgemv.STEP_ORDERED, wsgemv.STEP_ORDERED | wsgemv.STEP_FORCE_GRAPH, wsgemv.STEP_GROUPED,
                                  wsgemv.STEP_GROUPED | wsgemv.STEP_FORCE_GRAPH, wsgemv.STEP_GROUPED | wsgemv.STEP_EAGER])
def test_decode_step_takes_the_token(mode):
    """Replays with new activations each time: every replay's token is the
    argmax of that replay's logits (the token header clears itself)."""
    say(f"argmax step mode={mode:#x}")
    step_in = synth.decode_step_f16(workload=125, n_layers=1, lm_head_rows=100003)
    tok = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    val = torch.empty(1, device="cuda")
    lins, refs = _step_lins(step_in, tok, val)
    st = wsgemv.DecodeStep(lins, mode)
    lm = lins[-1]
    W = refs[-1][0]
    for rep in range(4):
        x = synth.f16_normal(126, rep, (lm.K,), synth.X_SIGMA)
        lm.x.copy_(dev(x))
        tok.fill_(-7)
        st()
        _check_fused(W, x, host(lm.y), int(host(tok)[0]), host(val), f"mode {mode:#x} replay {rep}")
    st.close()


def test_step_w8a8_token_and_split_ordered():
    """A W8A8 linear takes a token (the rescaled y), and an ORDERED fp16
    linear with a forced k-split takes it in the reduce."""
    say("argmax step w8a8 + split")
    N, K = 30000, 2048
    Wq = synth.int8_uniform(127, 0, (N, K))
    xq = synth.int8_uniform(127, 1, (K,))
    sw = synth.f32_uniform(127, 2, (N,), 0.001, 0.01)
    xs = torch.tensor([synth.X_SCALE_W8A8], device="cuda")
    y8 = torch.empty(N, device="cuda")
    t8 = torch.empty(1, dtype=torch.int32, device="cuda")
    W, x = _lm_case(20000, 3072, workload=128)
    y16 = torch.empty(20000, device="cuda")
    t16 = torch.empty(1, dtype=torch.int32, device="cuda")
    v16 = torch.empty(1, device="cuda")
    lins = [wsgemv.Linear(wsgemv.W8A8, dev(Wq), dev(xq), y8, N, K, scale=dev(sw), x_scale=xs, argmax_idx=t8),
            wsgemv.Linear(wsgemv.F16, dev(W), dev(x), y16, 20000, 3072, splits=3, argmax_idx=t16, argmax_val=v16)]
    for mode in (wsgemv.STEP_ORDERED, wsgemv.STEP_GROUPED | wsgemv.STEP_FORCE_GRAPH):
        use = lins if mode == wsgemv.STEP_ORDERED else lins[:1]
        st = wsgemv.DecodeStep(use, mode)
        st()
        st()
        acc_ref, y_ref, A = oracle.gemv_w8a8(Wq, sw, xq, synth.X_SCALE_W8A8)
        yh = host(y8)
        assert_within(yh, y_ref, A, "w8a8")
        t = int(host(t8)[0])
        assert t == oracle.argmax_f32(yh) and oracle.argmax_is_valid(t, y_ref, A)
        if mode == wsgemv.STEP_ORDERED:
            _check_fused(W, x, host(y16), int(host(t16)[0]), host(v16), "ordered split")
        st.close()


def _w4_aligned_row(x, K):
    """Canonical int4 words of a row whose weights follow the sign of x
    (q = 15 where x > 0, q = 0 elsewhere): a logit far above the others."""
    q = np.where(np.asarray(x, np.float32).reshape(-1) > 0, 15, 0).astype(np.uint32)
    words = np.zeros(K // 8, np.uint32)
    for i in range(8):
        words |= q[i::8] << (4 * i)
    return words


@pytest.mark.parametrize("kind,M", [(wsgemv.W4A16, 1), (wsgemv.W4A16, 3), (wsgemv.W4A16, 4), (wsgemv.W4A16, 8),
                                    (wsgemv.W4A8, 1)])
@pytest.mark.parametrize("mode,splits", [(wsgemv.STEP_ORDERED, 0), (wsgemv.STEP_ORDERED, 2),
                                         (wsgemv.STEP_GROUPED, 0),
                                         (wsgemv.STEP_GROUPED | wsgemv.STEP_FORCE_GRAPH, 0)])
def test_int4_tokens_per_position(kind, M, mode, splits):
    """An int4 lm_head-shaped linear takes one token per output row (for a
    verify block: per drafted position), with a planted maximum in one
    position and a bit-identical copy of it at a lower row (the tie)."""
    say(f"argmax int4 kind={kind} M={M} mode={mode:#x} S={splits}")
    N, K = 60001, 1024
    Wc = synth.w4_words(160, M, N, K)
    s4 = synth.f16_uniform(160, M + 1, (N, K // 128), 0.002, 0.02)
    X = synth.f16_normal(160, M + 2, (M, K), synth.X_SIGMA)
    Wc[40000] = _w4_aligned_row(X[M - 1], K)       # position M-1: planted maximum ...
    s4[40000] = np.float16(0.02)
    Wc[777], s4[777] = Wc[40000], s4[40000]         # ... and its copy at a lower row
    Wp, Sp = wsgemv.pack_w4(dev(Wc), dev(s4))
    y = torch.full((M, N), float("nan"), device="cuda")
    tok = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    val = torch.empty(M, device="cuda")
    x_d = dev(X) if kind == wsgemv.W4A16 else dev(X.reshape(K))
    lin = wsgemv.Linear(kind, Wp, x_d, y, N, K, M=M, scale=Sp, group=128, splits=splits, argmax_idx=tok,
                        argmax_val=val)
    st = wsgemv.DecodeStep([lin], mode)
    st()
    st()
    yh = host(y).reshape(M, N)
    if kind == wsgemv.W4A16:
        Y_ref, A = oracle.gemv_w4a16(Wc, s4, X)
        Y_ref, A = Y_ref.reshape(M, N), A.reshape(M, N)
    else:
        xq, sx = oracle.quantize_x_i8(X.reshape(K))
        Y_ref, A = oracle.gemv_w4a8(Wc, s4, xq, sx)
        Y_ref, A = Y_ref.reshape(1, N), A.reshape(1, N)
    assert_within(yh, Y_ref, A, "logits")
    toks, vals = host(tok), host(val)
    for m in range(M):
        t = int(toks[m])
        assert t == oracle.argmax_f32(yh[m]), f"position {m}: not the argmax of the kernel's logits"
        assert oracle.argmax_is_valid(t, Y_ref[m], A[m]), f"position {m}: not a largest exact logit"
        assert vals[m] == yh[m, t]
    assert int(toks[M - 1]) == 777                  # the tie goes to the lower row
    st.close()


def test_int4_tokens_k_zero():
    say("argmax int4 K=0")
    M, N = 3, 500
    y = torch.full((M, N), 5.0, device="cuda")
    tok = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    lin = wsgemv.Linear(wsgemv.W4A16, torch.empty(16, dtype=torch.uint8, device="cuda"),
                        torch.empty((M, 0), dtype=torch.float16, device="cuda"), y, N, 0, M=M,
                        scale=torch.empty(16, dtype=torch.uint8, device="cuda"), group=128, argmax_idx=tok)
    st = wsgemv.DecodeStep([lin], wsgemv.STEP_ORDERED)
    st()
    assert host(tok).tolist() == [0] * M and not host(y).any()
    st.close()
