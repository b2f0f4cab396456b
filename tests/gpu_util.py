"""Helpers shared by the GPU parity tests: host <-> device copies and the
parity assertions.  Expected values always come from the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle


def say(msg: str) -> None:
    """Name the case before the GPU runs it (flushed, so a crash still shows it)."""
    sys.stdout.write(f"[gpu-case] {msg}\n")
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def assert_within(y_gpu, y_ref, A, what: str = "") -> float:
    r = oracle.max_err_ratio(y_gpu, y_ref, A)
    assert r <= 1.0, f"{what}: max |err| / (1e-3 A + 1e-6) = {r:.3g}"
    return r


def assert_bits_equal(a: np.ndarray, b: np.ndarray, what: str = "") -> None:
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    assert a.shape == b.shape, (a.shape, b.shape)
    if not np.array_equal(a.view(np.uint8), b.view(np.uint8)):
        bad = np.flatnonzero(a.reshape(-1).view(np.uint32) != b.reshape(-1).view(np.uint32))
        raise AssertionError(f"{what}: {bad.size} elements differ, first at {bad[:5]}")
