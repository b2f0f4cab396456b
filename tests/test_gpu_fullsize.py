"""The full int4 decode steps at their real sizes, in the launch
configuration the benchmark times (the GROUPED plan): 28 layers x {qkv,
o, gate_up, down} + the 248320 x 1024 lm_head, at M = 1, at M = 4 and
M = 8 verify blocks, and with int8 activations.  Every linear is checked against
the oracle on sampled rows (the first and last rows and a seeded sample),
which the oracle computes one by one on the same inputs."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_within, dev, host, say
from weight_streaming_gemv_decode_amd import synth, wsgemv

pytestmark = pytest.mark.gpu


def _rows(N, name, k=48):
    r = synth.rng(150, sum(map(ord, name)) + N)
    pick = r.choice(N, size=min(N, k if name != "lm_head" else 1024), replace=False)
    return np.unique(np.concatenate([pick, [0, N - 1]]))


@pytest.fixture(scope="module", params=[1, 4, 8], ids=["M1", "M4", "M8"])
def w4_step(request):
    M = request.param
    return M, synth.decode_step_w4(workload=5, M=M)


def test_w4a16_full_step_grouped(w4_step):
    M, step_in = w4_step
    say(f"full W4A16 step M={M}, GROUPED")
    lins = []
    for name, Wc, s4, X in step_in:
        N, K = Wc.shape[0], Wc.shape[1] * 8
        Wp, Sp = wsgemv.pack_w4(dev(Wc), dev(s4))
        y = torch.full((M, N), float("nan"), device="cuda")
        lins.append(wsgemv.Linear(wsgemv.W4A16, Wp, dev(X), y, N, K, M=M, scale=Sp, group=128))
    st = wsgemv.DecodeStep(lins, wsgemv.STEP_GROUPED)
    st()
    for (name, Wc, s4, X), l in zip(step_in, lins):
        rows = _rows(Wc.shape[0], name)
        Y_ref, A = oracle.gemv_w4a16(Wc[rows], s4[rows], X)
        Y = host(l.y).reshape(M, -1)[:, rows]
        assert_within(Y, Y_ref.reshape(M, -1), A.reshape(M, -1), f"{name} M={M}")
        assert np.all(np.isfinite(host(l.y))), f"{name}: unwritten outputs"
    st.close()


def test_w4a8_full_step_grouped():
    say("full W4A8 step, GROUPED")
    step_in = synth.decode_step_w4(workload=5, M=1)
    lins = []
    for name, Wc, s4, X in step_in:
        N, K = Wc.shape[0], Wc.shape[1] * 8
        Wp, Sp = wsgemv.pack_w4(dev(Wc), dev(s4))
        y = torch.full((N,), float("nan"), device="cuda")
        lins.append(wsgemv.Linear(wsgemv.W4A8, Wp, dev(X.reshape(K)), y, N, K, scale=Sp, group=128))
    st = wsgemv.DecodeStep(lins, wsgemv.STEP_GROUPED)
    st()
    for (name, Wc, s4, X), l in zip(step_in, lins):
        rows = _rows(Wc.shape[0], name)
        xq, sx = oracle.quantize_x_i8(X.reshape(-1))
        y_ref, A = oracle.gemv_w4a8(Wc[rows], s4[rows], xq, sx)
        yh = host(l.y)
        assert_within(yh[rows], y_ref, A, name)
        assert np.all(np.isfinite(yh)), f"{name}: unwritten outputs"
    st.close()
