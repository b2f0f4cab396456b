"""Top-k on the GPU (wsg_topk_f32): the k indices must equal the oracle's
top-k of the same fp32 vector bit for bit (the order is total, so the
answer is unique), and the values must be the vector's own."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import dev, host, say
from weight_streaming_gemv_decode_amd import synth, wsgemv

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _topk(y, k, ws=None):
    idx = torch.full((k,), -7, dtype=torch.int32, device="cuda")
    val = torch.full((k,), 1234.0, device="cuda")
    wsgemv.topk_f32(dev(y), k, idx=idx, val=val, ws=ws)
    return host(idx).astype(np.int64), host(val)


def _check(y, k, what):
    got, vals = _topk(y, k)
    want = oracle.topk_f32(y, k)
    assert np.array_equal(got, want), f"{what}: first difference at {np.flatnonzero(got != want)[:3]}"
    exp = y[want].copy()
    exp[exp == 0] = 0.0                          # a -0 comes back as +0
    same = (vals.view(np.uint32) == exp.view(np.uint32)) | (np.isnan(vals) & np.isnan(exp))
    assert same.all(), f"{what}: values"


def test_golden():
    say("topk golden")
    g = json.load(open(os.path.join(GOLDEN, "topk_order.json")))
    for c in g["cases"]:
        y = np.array([int(v, 16) for v in c["bits"]], np.uint32).view(np.float32)
        got, _ = _topk(y, c["k"])
        assert got.tolist() == c["topk"], c["note"]


# 16 / 17 / 33 / 256 lists of 1024 candidates: one merging workgroup; one
# merging group of 17; groups of 32 with a last group of one list; eight
# full groups
@pytest.mark.parametrize("N", [1, 64, 1023, 1024, 1025, 2049, 16384, 16385, 32769, 248320, 262144,
                               (1 << 20) + 7])
@pytest.mark.parametrize("k", [1, 2, 8, 50, 64])
def test_random_with_ties_nan_and_signed_zero(N, k):
    if k > N:
        pytest.skip("k > N")
    say(f"topk N={N} k={k}")
    r = synth.rng(170, N + k)
    y = np.round(r.normal(0, 30, N)).astype(np.float32)      # integers: many exact ties
    y[r.integers(0, N, max(1, N // 50))] = -0.0
    if N > 100:
        y[r.integers(0, N, N // 100)] = np.nan
        top = np.nanmax(y)
        y[r.choice(N, min(N, 5), replace=False)] = top + 1   # five equal maxima
    _check(y, k, f"N={N} k={k}")


def test_several_selection_passes():
    """3,000,000 values with k = 64: the first pass leaves 2,930 lists
    (187,520 candidates), more than the merge takes, so a second pass runs
    before it."""
    say("topk multi-pass")
    N, k = 3_000_000, 64
    r = synth.rng(171, 0)
    y = r.normal(0, 1, N).astype(np.float32)
    y[r.integers(0, N, 1000)] = 3.5                           # ties among the top values
    _check(y, k, "multi-pass")


def test_k_equals_n_and_constant_vectors():
    say("topk k=N, constant")
    _check(np.array([5, -1, 5, 2], np.float32), 4, "k=N")
    _check(np.full(5000, 2.0, np.float32), 64, "all equal")
    _check(np.full(5000, np.nan, np.float32), 10, "all NaN")


def test_workspace_contents_do_not_matter():
    say("topk ws garbage")
    N, k = 300000, 50
    ws = torch.full((wsgemv.lib().wsg_topk_ws_bytes(N, k),), 0xFF, dtype=torch.uint8, device="cuda")
    r = synth.rng(172, 0)
    for rep in range(3):
        y = r.normal(0, 1, N).astype(np.float32)
        got, _ = _topk(y, k, ws=ws)
        assert np.array_equal(got, oracle.topk_f32(y, k)), rep


def test_topk_of_gemv_logits_matches_token():
    """Top-k over the logits the fused lm_head GEMV wrote: its first entry
    is the fused greedy token."""
    say("topk of lm_head logits")
    N, K = 100000, 1024
    W = synth.f16_normal(173, 0, (N, K), synth.W_SIGMA)
    x = synth.f16_normal(173, 1, (K,), synth.X_SIGMA)
    y, tok = wsgemv.gemv_f16_argmax(dev(W), dev(x))
    idx, _ = wsgemv.topk_f32(y, 50)
    yh = host(y)
    assert int(host(idx)[0]) == int(host(tok)[0])
    assert np.array_equal(host(idx).astype(np.int64), oracle.topk_f32(yh, 50))
