"""CPU oracle for the batch-1 decode GEMV (y = W . x) and its quantised forms.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers.  The GPU library never
imports or loads anything from here, and nothing here imports the library.

The arithmetic lives in ``oracle.c`` (plain C, fp64 sums of exactly decoded
fp16 values, exact int64 sums for int8; see that file for the passages of
the pages each function follows).  This module only marshals numpy arrays
through ctypes and states the parity rule.

Parity rule for floating point, per output element:
    |y_hat - y| <= 1e-3 * A + 1e-6,   A = sum_k |w_k * x_k|
and bit-exact equality for the int32 accumulators of the int8 path.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

REL_TOL = 1e-3
ABS_TOL = 1e-6

ERR_NONFINITE = 1
ERR_SHAPE = 2
ERR_RANGE = 3


class OracleError(RuntimeError):
    pass


def build(out_path: str = _LIB_PATH, defines: Sequence[str] = (), extra: Sequence[str] = ()) -> str:
    """Compile oracle.c with gcc (no fused multiply-add, no fast-math);
    `extra` adds compiler flags (the tests' sanitizer build)."""
    tmp = out_path + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c99",
           "-Wall", "-shared", "-fPIC", *extra, *[f"-D{d}" for d in defines], _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.orc_f16_decode.argtypes = [P, I64, P]
    lib.orc_gemv_f16.argtypes = [P, P, I64, I64, P, P]
    lib.orc_gemv_w8a8.argtypes = [P, P, P, ctypes.c_float, I64, I64, P, P, P]
    lib.orc_gemv_w4a16.argtypes = [P, P, P, I64, I64, I64, I64, P, P]
    lib.orc_quantize_x_i8.argtypes = [P, I64, P, P]
    lib.orc_gemv_w4a8.argtypes = [P, P, P, ctypes.c_float, I64, I64, I64, P, P]
    lib.orc_argmax_f32.argtypes = [P, I64, P]
    lib.orc_round_f16.argtypes = [P, I64, P]
    lib.orc_causal_conv1d_step.argtypes = [P, P, P, P, I64, I64, ctypes.c_int, P, P]
    lib.orc_topk_f32.argtypes = [P, I64, I64, P]
    for f in (lib.orc_topk_f32, lib.orc_causal_conv1d_step, lib.orc_f16_decode, lib.orc_gemv_f16, lib.orc_gemv_w8a8, lib.orc_gemv_w4a16,
              lib.orc_quantize_x_i8, lib.orc_gemv_w4a8, lib.orc_argmax_f32, lib.orc_round_f16):
        f.restype = ctypes.c_int
    lib.orc_set_threads.argtypes = [ctypes.c_int]
    lib.orc_set_threads.restype = None
    lib.orc_max_threads.argtypes = []
    lib.orc_max_threads.restype = ctypes.c_int
    return lib


_lib: Optional[ctypes.CDLL] = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the compiled oracle, building it first only if it is absent."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        alt = os.environ.get("WSG_ORACLE_LIB")  # another build of the same source (the tests' sanitizer build)
        if alt:
            _lib = _bind(ctypes.CDLL(alt))
            return _lib
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check(code: int, what: str) -> None:
    if code != 0:
        raise OracleError(f"{what}: oracle status {code}")


def set_threads(n: int, lib: Optional[ctypes.CDLL] = None) -> None:
    (lib or load()).orc_set_threads(int(n))


def max_threads(lib: Optional[ctypes.CDLL] = None) -> int:
    return int((lib or load()).orc_max_threads())


def f16_decode(h: np.ndarray, lib: Optional[ctypes.CDLL] = None) -> np.ndarray:
    """Exact fp16 -> float64 from the bit pattern (uint16 or float16 input)."""
    bits = np.ascontiguousarray(np.asarray(h).view(np.uint16) if np.asarray(h).dtype == np.float16
                                else np.asarray(h, dtype=np.uint16))
    out = np.empty(bits.shape, dtype=np.float64)
    _check((lib or load()).orc_f16_decode(_ptr(bits), bits.size, _ptr(out)), "f16_decode")
    return out


def _u16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError(f"expected float16 or uint16 bit patterns, got {a.dtype}")
    return a


def gemv_f16(W: np.ndarray, x: np.ndarray, lib: Optional[ctypes.CDLL] = None
             ) -> Tuple[np.ndarray, np.ndarray]:
    """(y, A) for y = W . x with W fp16 [N, K] and x fp16 [K]."""
    W = _u16(W)
    x = _u16(x)
    N, K = W.shape
    if x.shape != (K,):
        raise ValueError("x must have shape (K,)")
    y = np.empty(N, np.float64)
    A = np.empty(N, np.float64)
    _check((lib or load()).orc_gemv_f16(_ptr(W), _ptr(x), N, K, _ptr(y), _ptr(A)), "gemv_f16")
    return y, A


def gemv_w8a8(Wq: np.ndarray, w_scale: np.ndarray, xq: np.ndarray, x_scale: float,
              lib: Optional[ctypes.CDLL] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(acc int32, y float64, A) for the int8 weight x int8 activation product."""
    Wq = np.ascontiguousarray(Wq, dtype=np.int8)
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    w_scale = np.ascontiguousarray(w_scale, dtype=np.float32)
    N, K = Wq.shape
    if xq.shape != (K,) or w_scale.shape != (N,):
        raise ValueError("shape mismatch")
    acc = np.empty(N, np.int32)
    y = np.empty(N, np.float64)
    A = np.empty(N, np.float64)
    _check((lib or load()).orc_gemv_w8a8(_ptr(Wq), _ptr(w_scale), _ptr(xq), float(np.float32(x_scale)),
                                         N, K, _ptr(acc), _ptr(y), _ptr(A)), "gemv_w8a8")
    return acc, y, A


def gemv_w4a16(Wc: np.ndarray, s4: np.ndarray, X: np.ndarray, group: int = 128,
               lib: Optional[ctypes.CDLL] = None) -> Tuple[np.ndarray, np.ndarray]:
    """(Y, A) for canonical int4 words Wc uint32 [N, K/8], fp16 scales
    s4 [N, K/group] and fp16 activations X [M, K] (or [K] for M = 1)."""
    Wc = np.ascontiguousarray(Wc, dtype=np.uint32)
    s4 = _u16(s4)
    X = _u16(X)
    squeeze = X.ndim == 1
    if squeeze:
        X = X.reshape(1, -1)
    M, K = X.shape
    N = Wc.shape[0]
    if Wc.shape != (N, K // 8) or s4.shape != (N, K // group):
        raise ValueError("shape mismatch")
    Y = np.empty((M, N), np.float64)
    A = np.empty((M, N), np.float64)
    _check((lib or load()).orc_gemv_w4a16(_ptr(Wc), _ptr(s4), _ptr(X), M, N, K, group,
                                          _ptr(Y), _ptr(A)), "gemv_w4a16")
    if squeeze:
        return Y[0], A[0]
    return Y, A


def quantize_x_i8(x: np.ndarray, lib: Optional[ctypes.CDLL] = None) -> Tuple[np.ndarray, np.float32]:
    """(xq int8 [K], s_x fp32): per-token symmetric int8 quantisation of fp16 x."""
    x = _u16(x)
    K = x.shape[0]
    xq = np.empty(K, np.int8)
    sx = np.empty(1, np.float32)
    _check((lib or load()).orc_quantize_x_i8(_ptr(x), K, _ptr(xq), _ptr(sx)), "quantize_x_i8")
    return xq, sx[0]


def gemv_w4a8(Wc: np.ndarray, s4: np.ndarray, xq: np.ndarray, s_x: float, group: int = 128,
              lib: Optional[ctypes.CDLL] = None) -> Tuple[np.ndarray, np.ndarray]:
    """(y, A) for canonical int4 words times int8 activations xq with scale s_x."""
    Wc = np.ascontiguousarray(Wc, dtype=np.uint32)
    s4 = _u16(s4)
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    N = Wc.shape[0]
    K = xq.shape[0]
    if Wc.shape != (N, K // 8) or s4.shape != (N, K // group):
        raise ValueError("shape mismatch")
    y = np.empty(N, np.float64)
    A = np.empty(N, np.float64)
    _check((lib or load()).orc_gemv_w4a8(_ptr(Wc), _ptr(s4), _ptr(xq), float(np.float32(s_x)), N, K, group,
                                         _ptr(y), _ptr(A)), "gemv_w4a8")
    return y, A


def causal_conv1d_step(x: np.ndarray, w: np.ndarray, bias: Optional[np.ndarray], state: np.ndarray,
                       silu: bool, lib: Optional[ctypes.CDLL] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(out float64 [C], A [C], new state fp32 [C, W-1]) for one decode step
    of the causal depthwise conv: x fp32 [C], w fp16 [C, W], bias fp32 [C]
    or None, state fp32 [C, W-1] (oldest first; not modified)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    w = _u16(w)
    C, W = w.shape
    st = np.ascontiguousarray(state, dtype=np.float32).copy()
    if x.shape != (C,) or st.shape != (C, W - 1):
        raise ValueError("shape mismatch")
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty(C, np.float64)
    A = np.empty(C, np.float64)
    _check((lib or load()).orc_causal_conv1d_step(_ptr(x), _ptr(w), None if b is None else _ptr(b), _ptr(st), C, W,
                                                  int(bool(silu)), _ptr(out), _ptr(A)), "causal_conv1d_step")
    return out, A, st


def conv_bound(A: np.ndarray, out: np.ndarray, silu: bool) -> np.ndarray:
    """Tolerance of the conv step: the GEMV rule on the pre-activation sum;
    SiLU (slope at most 1.1) carries it over, plus a relative term for the
    fp32 exponential and division."""
    A = np.asarray(A, np.float64)
    if not silu:
        return bound(A)
    return REL_TOL * (1.1 * A + np.abs(np.asarray(out, np.float64))) + ABS_TOL


def round_f16(v: np.ndarray, lib: Optional[ctypes.CDLL] = None) -> np.ndarray:
    """Round doubles to IEEE binary16 (nearest, ties to even); returns float16."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    _check((lib or load()).orc_round_f16(_ptr(v), v.size, _ptr(out)), "round_f16")
    return out.view(np.float16)


def chain_f16(Ws: Sequence[np.ndarray], x0: np.ndarray, lib: Optional[ctypes.CDLL] = None
              ) -> List[Tuple[np.ndarray, np.ndarray]]:
    """A chain of linears where each one's fp16-rounded output is the next
    one's input: returns [(y_i float64, y16_i float16)] for i = 0..len-1."""
    out = []
    x = np.asarray(x0, np.float16)
    for W in Ws:
        y, _ = gemv_f16(W, x, lib)
        x = round_f16(y, lib)
        out.append((y, x))
    return out


def argmax_f32(y: np.ndarray, lib: Optional[ctypes.CDLL] = None) -> int:
    """Index of the largest fp32 value: IEEE comparison (-0 == +0), NaN below
    every number, lowest index on ties.  This is the greedy token choice."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    if y.ndim != 1:
        raise ValueError("y must be one-dimensional")
    out = np.zeros(1, np.int64)
    _check((lib or load()).orc_argmax_f32(_ptr(y), y.size, _ptr(out)), "argmax_f32")
    return int(out[0])


def topk_f32(y: np.ndarray, k: int, lib: Optional[ctypes.CDLL] = None) -> np.ndarray:
    """Indices of the k largest fp32 values in the greedy token's order
    (larger first, NaN below every number, -0 == +0, lower index first
    among equals), as int64 [k]."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.zeros(k, np.int64)
    _check((lib or load()).orc_topk_f32(_ptr(y), y.size, int(k), _ptr(out)), "topk_f32")
    return out


def argmax_is_valid(idx: int, y_ref: np.ndarray, A: np.ndarray) -> bool:
    """True when token idx is a largest logit of the exact product within
    the parity bound: no exact logit exceeds y_ref[idx] by more than the
    two elements' bounds allow (the GPU's fp32 logits may order near-equal
    values differently from the exact ones, never far-apart ones)."""
    y_ref = np.asarray(y_ref, np.float64)
    b = bound(A)
    return bool(np.all(y_ref - b <= y_ref[idx] + b[idx]))


def decode_step_f16(linears: Iterable[Tuple[np.ndarray, np.ndarray]],
                    lib: Optional[ctypes.CDLL] = None) -> List[Tuple[np.ndarray, np.ndarray]]:
    """The decode step is the per-linear product on each (W, x) pair."""
    return [gemv_f16(W, x, lib) for W, x in linears]


def bound(A: np.ndarray) -> np.ndarray:
    return REL_TOL * np.asarray(A, np.float64) + ABS_TOL


def max_err_ratio(y_hat: np.ndarray, y: np.ndarray, A: np.ndarray) -> float:
    """max over elements of |y_hat - y| / (1e-3 A + 1e-6); parity iff <= 1."""
    err = np.abs(np.asarray(y_hat, np.float64) - np.asarray(y, np.float64))
    r = err / bound(A)
    if r.size == 0:
        return 0.0
    if not np.all(np.isfinite(r)):
        return float("inf")
    return float(r.max())
