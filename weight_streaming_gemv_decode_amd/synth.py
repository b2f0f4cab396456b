"""Seeded synthetic inputs for the batch-1 decode GEMV workloads.

This module draws random tensors and nothing else: it holds none of the
arithmetic of the method (no products, no dequantisation, no unpacking), so
both the CPU oracle and the HIP path can take their inputs from it without
sharing any computation.

Every tensor comes from its own numpy PCG64 stream seeded with the pair
``(workload_id, tensor_id)`` (a ``numpy.random.SeedSequence`` entropy list), so
any tensor can be regenerated alone and no two tensors share a stream.

Distributions (the pages give only the precisions; the shapes and
distributions below are the synthetic stand-ins for the pages' MiniCPM-V
decode weight stream, "FP16 weights" read once per step, and for the INT8 /
INT4 formats the pages name as the next step and as the Arm quantised paths):

* fp16 weights  ~ N(0, 0.02) (0.02 is the standard deviation), rounded to
  fp16 by numpy (round to nearest even); fp16 activations ~ N(0, 1).
* int8 weights and activations uniform on the integers [-127, 127].
* fp32 per-output-channel scales ~ U(0.001, 0.01); per-tensor scale 0.02.
* int4 weights: canonical ``uint32[N, K/8]`` words drawn uniformly on
  [0, 2**32).  Every 4-bit field of a uniform 32-bit word is itself uniform
  on 0..15 and independent of the others, which is exactly "q uniform in
  0..15"; the field order inside a word (canonical: element k = 8*j + i in
  bits [4i, 4i+3] of word j) is a reading of the format, fixed by the
  consumers, not by this generator.
* fp16 group scales ~ U(0.002, 0.02), one per 128 consecutive k of a row.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple

import numpy as np

__all__ = [
    "rng", "f16_normal", "int8_uniform", "f32_uniform", "f16_uniform",
    "w4_words", "LinearShape", "DECODE_LAYER", "decode_step_shapes",
    "W_SIGMA", "X_SIGMA", "X_SCALE_W8A8", "LMHEAD", "C1_SHAPE", "C4_SHAPES",
    "N_LAYERS", "GROUP",
]

# Workload constants: sizes of a small decoder with a ~248k vocabulary.
W_SIGMA = 0.02
X_SIGMA = 1.0
X_SCALE_W8A8 = 0.02
GROUP = 128
N_LAYERS = 28
C1_SHAPE = (2048, 2048)
LMHEAD = (248320, 1024)
C4_SHAPES = ((14336, 4096), (4096, 14336))


@dataclasses.dataclass(frozen=True)
class LinearShape:
    name: str
    N: int
    K: int


# One decoder layer: fused q/k/v projection, output projection, fused
# gate+up projection and down projection, hidden size 1024.
DECODE_LAYER: Tuple[LinearShape, ...] = (
    LinearShape("qkv", 2048, 1024),
    LinearShape("o", 1024, 1024),
    LinearShape("gate_up", 6144, 1024),
    LinearShape("down", 1024, 3072),
)


def decode_step_shapes(n_layers: int = N_LAYERS) -> List[Tuple[str, int, int, int, int]]:
    """(name, N, K, w_tensor_id, x_tensor_id) for every linear of one step.

    Layer l uses weight ids 8l+0..3 and activation ids 8l+4..7 in the order
    of DECODE_LAYER; the lm_head uses ids 1000 (weight) and 1001 (x).
    """
    out = []
    for layer in range(n_layers):
        for j, s in enumerate(DECODE_LAYER):
            out.append((f"L{layer}.{s.name}", s.N, s.K, 8 * layer + j, 8 * layer + 4 + j))
    out.append(("lm_head", LMHEAD[0], LMHEAD[1], 1000, 1001))
    return out


def rng(workload: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng([int(workload), int(tensor)])


def f16_normal(workload: int, tensor: int, shape, sigma: float) -> np.ndarray:
    g = rng(workload, tensor)
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(sigma)).astype(np.float16)


def int8_uniform(workload: int, tensor: int, shape) -> np.ndarray:
    return rng(workload, tensor).integers(-127, 128, shape, dtype=np.int8)


def f32_uniform(workload: int, tensor: int, shape, lo: float, hi: float) -> np.ndarray:
    return rng(workload, tensor).uniform(lo, hi, shape).astype(np.float32)


def f16_uniform(workload: int, tensor: int, shape, lo: float, hi: float) -> np.ndarray:
    return rng(workload, tensor).uniform(lo, hi, shape).astype(np.float16)


def w4_words(workload: int, tensor: int, N: int, K: int) -> np.ndarray:
    """Canonical int4 weights as uint32[N, K/8] (K must be a multiple of 8)."""
    if K % 8:
        raise ValueError("K must be a multiple of 8 for packed int4 rows")
    return rng(workload, tensor).integers(0, 2 ** 32, (N, K // 8), dtype=np.uint32)


def workload_tensors_f16(workload: int, N: int, K: int, w_id: int = 0, x_id: int = 1) -> Dict[str, np.ndarray]:
    return {"W": f16_normal(workload, w_id, (N, K), W_SIGMA),
            "x": f16_normal(workload, x_id, (K,), X_SIGMA)}


def decode_step_f16(workload: int = 3, n_layers: int = N_LAYERS, lm_head_rows: int = LMHEAD[0],
                    threads: int = 8):
    """[(name, W fp16 [N,K], x fp16 [K])] for every linear of one step, each
    tensor from its own stream (generated in parallel; the result does not
    depend on the thread count)."""
    from concurrent.futures import ThreadPoolExecutor
    shapes = decode_step_shapes(n_layers)
    shapes = [(n, (lm_head_rows if n == "lm_head" else N), K, wi, xi) for n, N, K, wi, xi in shapes]

    def gen(s):
        name, N, K, wi, xi = s
        return name, f16_normal(workload, wi, (N, K), W_SIGMA), f16_normal(workload, xi, (K,), X_SIGMA)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        return list(ex.map(gen, shapes))


def decode_step_w4(workload: int = 5, n_layers: int = N_LAYERS, lm_head_rows: int = LMHEAD[0], M: int = 1,
                   threads: int = 8):
    """[(name, Wc uint32 [N,K/8], s4 fp16 [N,K/128], X fp16 [M,K])] for one step."""
    from concurrent.futures import ThreadPoolExecutor
    shapes = decode_step_shapes(n_layers)
    shapes = [(n, (lm_head_rows if n == "lm_head" else N), K, wi, xi) for n, N, K, wi, xi in shapes]

    def gen(s):
        name, N, K, wi, xi = s
        X = f16_normal(workload, xi if M == 1 else 2000 + xi, (M, K), X_SIGMA)
        return (name, w4_words(workload, wi, N, K),
                f16_uniform(workload, 500 + wi, (N, K // GROUP), 0.002, 0.02), X)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        return list(ex.map(gen, shapes))
