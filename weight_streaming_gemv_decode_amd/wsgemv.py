"""ctypes binding of libwsgemv.so (the C ABI in include/wsgemv.h).

Argument marshalling only: every function checks dtype, device, shape and
contiguity of torch tensors, passes their device pointers and the current
torch stream to the library, and turns a non-zero status into WsgError.  All
arithmetic runs in the library's HIP kernels.  There is no fallback: if the
library is missing or cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import List, Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# another build of the same sources may be named by WSGEMV_LIB (the tests' host-sanitizer build)
LIB_PATH = os.environ.get("WSGEMV_LIB") or os.path.join(_HERE, "libwsgemv.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "wsgemv.h")

F16, W8A8, W4A16, W4A8, W8A8_DYN = 0, 1, 2, 3, 4
ARGMAX_WS_BYTES, WITH_ARGMAX, TOPK_MAX = 8192, 0x100, 64
STATIC_SCRATCH_BYTES = 16 << 20
STEP_ORDERED, STEP_GROUPED, STEP_PERSISTENT, STEP_EAGER, STEP_FORCE_GRAPH = 0, 1, 2, 0x100, 0x200
STEP_GRAPH_MIN_LAUNCHES = 8
STATUS = {0: "WSG_OK", 1: "WSG_ERR_NULL", 2: "WSG_ERR_SHAPE", 3: "WSG_ERR_ALIGN", 4: "WSG_ERR_UNSUPPORTED",
          5: "WSG_ERR_WORKSPACE", 6: "WSG_ERR_HIP", 7: "WSG_ERR_NOMEM", 8: "WSG_ERR_STATE"}


class WsgError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str = ""):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({detail})")


class wsg_linear(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("M", ctypes.c_int32), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("W", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("x", ctypes.c_void_p),
                ("x_scale", ctypes.c_void_p), ("y", ctypes.c_void_p), ("acc_out", ctypes.c_void_p),
                ("group", ctypes.c_int32), ("splits", ctypes.c_int32), ("argmax_idx", ctypes.c_void_p),
                ("argmax_val", ctypes.c_void_p), ("conv_w", ctypes.c_void_p), ("conv_bias", ctypes.c_void_p),
                ("conv_state", ctypes.c_void_p), ("conv_out", ctypes.c_void_p), ("conv_width", ctypes.c_int32),
                ("conv_silu", ctypes.c_int32), ("y16", ctypes.c_void_p)]


_lib: Optional[ctypes.CDLL] = None


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "wsg_status_string": ([I32], ctypes.c_char_p),
        "wsg_last_hip_error": ([], I32),
        "wsg_build_info": ([], ctypes.c_char_p),
        "wsg_plan_splits": ([I32, I64, I64, I64], I32),
        "wsg_workspace_bytes": ([I32, I64, I64, I64, I32], SZ),
        "gemv_f16": ([P, P, P, I64, I64, I32, P, SZ, P], I32),
        "gemv_f16_static": ([P, P, P, I64, I64, I32, P], I32),
        "gemv_w8a8": ([P, P, P, P, P, P, I64, I64, I32, P, SZ, P], I32),
        "wsg_w4_packed_weight_bytes": ([I64, I64], SZ),
        "wsg_w4_packed_scale_bytes": ([I64, I64, I64], SZ),
        "wsg_pack_w4": ([P, P, P, P, I64, I64, I64, P], I32),
        "gemv_w4a16": ([P, P, P, P, I64, I64, I64, I64, I32, P, SZ, P], I32),
        "gemv_w4a8": ([P, P, P, P, P, P, I64, I64, I64, I32, P, SZ, P], I32),
        "gemv_w8a8_dyn": ([P, P, P, P, P, P, P, I64, I64, I32, P, SZ, P], I32),
        "wsg_argmax_f32": ([P, I64, P, P, P, SZ, P], I32),
        "gemv_f16_argmax": ([P, P, P, P, P, I64, I64, I32, P, SZ, P], I32),
        "causal_conv1d_step": ([P, P, P, P, P, I64, I32, I32, P], I32),
        "wsg_topk_ws_bytes": ([I64, I32], SZ),
        "wsg_topk_f32": ([P, I64, I32, P, P, P, SZ, P], I32),
        "wsg_decode_step_create": ([ctypes.POINTER(wsg_linear), I32, I32, P, ctypes.POINTER(P)], I32),
        "decode_step_linears": ([P, P], I32),
        "wsg_decode_step_destroy": ([P], I32),
        "wsg_decode_step_info": ([P, ctypes.POINTER(I32), ctypes.POINTER(I64), ctypes.POINTER(I32)], I32),
        "wsg_decode_step_status": ([P, P, ctypes.POINTER(ctypes.c_uint32)], I32),
        "wsg_decode_step_trace": ([P, P, I64], I32),
        "wsg_chain_grid": ([I64, I32, I32, I32], I64),
        "wsg_test_set_fault": ([I32], I32),
        "wsg_test_live_blocks": ([], I64),
        "wsg_read_probe": ([P, SZ, P, I32, P], I32),
        "wsg_read_probe_grid": ([SZ], I32),
        "wsg_tune_set": ([ctypes.c_char_p, I64], I32),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    return lib


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m "
                               "weight_streaming_gemv_decode_amd.build` (there is no fallback path)")
        _lib = _bind(ctypes.CDLL(LIB_PATH))
    return _lib


def header_functions() -> List[str]:
    """Names of the functions include/wsgemv.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)))


def _check(status: int, what: str) -> None:
    if status != 0:
        detail = lib().wsg_status_string(status).decode()
        if status == 6:
            detail += f"; hipError_t {lib().wsg_last_hip_error()}"
        raise WsgError(status, what, detail)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t: torch.Tensor, dtype, name: str, shape=None) -> int:
    """Device pointer of t after checking its type, dtype, contiguity and
    shape, and last that it lives on a GPU."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    return t.data_ptr()


def _check_tensor(t, dtypes, name: str, numel: Optional[int] = None, min_bytes: Optional[int] = None,
                  optional: bool = False, device: bool = True) -> None:
    """Checks a tensor handed to a decode-step linear, in the same order as
    _dev: type, dtype, contiguity, size (an exact element count, or at least
    min_bytes bytes), then (device=True) that it lives on a GPU."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be one of {dtypes}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()} (shape {tuple(t.shape)})")
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise ValueError(f"{name} must hold at least {min_bytes} bytes, got {t.numel() * t.element_size()}")
    if device and t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")


def plan_splits(kind: int, M: int, N: int, K: int) -> int:
    return int(lib().wsg_plan_splits(kind, M, N, K))


def workspace_bytes(kind: int, M: int, N: int, K: int, splits: int = 0) -> int:
    return int(lib().wsg_workspace_bytes(kind, M, N, K, splits))


def workspace(kind: int, M: int, N: int, K: int, splits: int = 0, device="cuda") -> Optional[torch.Tensor]:
    n = workspace_bytes(kind, M, N, K, splits)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def _ws(ws: Optional[torch.Tensor]) -> Tuple[int, int]:
    if ws is None:
        return 0, 0
    if ws.device.type != "cuda" or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def gemv_f16(W: torch.Tensor, x: torch.Tensor, y: Optional[torch.Tensor] = None, splits: int = 0,
             ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y[n] = sum_k W[n,k] x[k]; W fp16 [N,K], x fp16 [K], y fp32 [N]."""
    N, K = W.shape
    if y is None:
        y = torch.empty(N, dtype=torch.float32, device=W.device)
    if ws is None:
        ws = workspace(F16, 1, N, K, splits, W.device)
    wp, wn = _ws(ws)
    _check(lib().gemv_f16(_dev(W, torch.float16, "W"), _dev(x, torch.float16, "x", (K,)),
                          _dev(y, torch.float32, "y", (N,)), N, K, splits, wp, wn, _stream(stream)), "gemv_f16")
    return y


def gemv_f16_static(W: torch.Tensor, x: torch.Tensor, y: torch.Tensor, splits: int = 0, stream=None) -> torch.Tensor:
    """gemv_f16 with no workspace: the library's per-GPU scratch array holds
    the split-K partials and the call allocates nothing.  Calls that overlap
    in time on one GPU race on that array."""
    N, K = W.shape
    _check(lib().gemv_f16_static(_dev(W, torch.float16, "W"), _dev(x, torch.float16, "x", (K,)),
                                 _dev(y, torch.float32, "y", (N,)), N, K, splits, _stream(stream)), "gemv_f16_static")
    return y


def argmax_f32(y: torch.Tensor, token: Optional[torch.Tensor] = None, token_logit: Optional[torch.Tensor] = None,
               ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Greedy token over fp32 y [N] (lowest index among the largest; NaN below
    every number); returns the int32 [1] token tensor."""
    N = y.shape[0]
    if token is None:
        token = torch.empty(1, dtype=torch.int32, device=y.device)
    if ws is None:
        ws = torch.empty(ARGMAX_WS_BYTES, dtype=torch.uint8, device=y.device)
    wp, wn = _ws(ws)
    tl = _dev(token_logit, torch.float32, "token_logit", (1,)) if token_logit is not None else None
    _check(lib().wsg_argmax_f32(_dev(y, torch.float32, "y", (N,)), N, _dev(token, torch.int32, "token", (1,)), tl,
                                wp, wn, _stream(stream)), "wsg_argmax_f32")
    return token


def topk_f32(y: torch.Tensor, k: int, idx: Optional[torch.Tensor] = None, val: Optional[torch.Tensor] = None,
             ws: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """(idx int32 [k], val): the k largest of fp32 y [N], larger first, lower index first among equals."""
    N = y.shape[0]
    if idx is None:
        idx = torch.empty(k, dtype=torch.int32, device=y.device)
    if ws is None:
        n = int(lib().wsg_topk_ws_bytes(N, k))
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=y.device)
    wp, wn = _ws(ws)
    vp = _dev(val, torch.float32, "val", (k,)) if val is not None else None
    _check(lib().wsg_topk_f32(_dev(y, torch.float32, "y", (N,)), N, k, _dev(idx, torch.int32, "idx", (k,)), vp, wp, wn,
                              _stream(stream)), "wsg_topk_f32")
    return idx, val


def gemv_f16_argmax(W: torch.Tensor, x: torch.Tensor, y: Optional[torch.Tensor] = None,
                    token: Optional[torch.Tensor] = None, token_logit: Optional[torch.Tensor] = None,
                    splits: int = 0, ws: Optional[torch.Tensor] = None, stream=None):
    """(y, token): the fp16 GEMV y = W . x with the greedy token over y fused in."""
    N, K = W.shape
    if y is None:
        y = torch.empty(N, dtype=torch.float32, device=W.device)
    if token is None:
        token = torch.empty(1, dtype=torch.int32, device=W.device)
    if ws is None:
        ws = workspace(F16 | WITH_ARGMAX, 1, N, K, splits, W.device)
    wp, wn = _ws(ws)
    tl = _dev(token_logit, torch.float32, "token_logit", (1,)) if token_logit is not None else None
    _check(lib().gemv_f16_argmax(_dev(W, torch.float16, "W"), _dev(x, torch.float16, "x", (K,)),
                                 _dev(y, torch.float32, "y", (N,)), _dev(token, torch.int32, "token", (1,)), tl,
                                 N, K, splits, wp, wn, _stream(stream)), "gemv_f16_argmax")
    return y, token


def causal_conv1d_step(x: torch.Tensor, w: torch.Tensor, state: torch.Tensor, bias: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None, silu: bool = False, stream=None) -> torch.Tensor:
    """One causal depthwise conv1d decode step: x fp32 [C], w fp16 [C, W], state fp32 [C, W-1]
    (updated in place), bias fp32 [C] or None; returns out fp32 [C]."""
    C, W = w.shape
    if out is None:
        out = torch.empty(C, dtype=torch.float32, device=x.device)
    bp = _dev(bias, torch.float32, "bias", (C,)) if bias is not None else None
    _check(lib().causal_conv1d_step(_dev(x, torch.float32, "x", (C,)), _dev(w, torch.float16, "w", (C, W)), bp,
                                    _dev(state, torch.float32, "state", (C, W - 1)),
                                    _dev(out, torch.float32, "out", (C,)), C, W, int(bool(silu)), _stream(stream)),
           "causal_conv1d_step")
    return out


def gemv_w8a8(Wq: torch.Tensor, w_scale: torch.Tensor, xq: torch.Tensor, x_scale: torch.Tensor,
              y: Optional[torch.Tensor] = None, acc_out: Optional[torch.Tensor] = None, want_acc: bool = True,
              splits: int = 0, ws: Optional[torch.Tensor] = None, stream=None):
    """(y, acc): acc[n] = sum_k Wq[n,k] xq[k] (int32), y = acc * w_scale[n] * x_scale."""
    N, K = Wq.shape
    if y is None:
        y = torch.empty(N, dtype=torch.float32, device=Wq.device)
    if acc_out is None and want_acc:
        acc_out = torch.empty(N, dtype=torch.int32, device=Wq.device)
    if ws is None:
        ws = workspace(W8A8, 1, N, K, splits, Wq.device)
    wp, wn = _ws(ws)
    acc_p = _dev(acc_out, torch.int32, "acc_out", (N,)) if acc_out is not None else None
    _check(lib().gemv_w8a8(_dev(Wq, torch.int8, "Wq"), _dev(w_scale, torch.float32, "w_scale", (N,)),
                           _dev(xq, torch.int8, "xq", (K,)), _dev(x_scale, torch.float32, "x_scale", (1,)),
                           _dev(y, torch.float32, "y", (N,)), acc_p, N, K, splits, wp, wn, _stream(stream)),
           "gemv_w8a8")
    return y, acc_out


def gemv_w8a8_dyn(Wq: torch.Tensor, w_scale: torch.Tensor, x: torch.Tensor, y: Optional[torch.Tensor] = None,
                  acc_out: Optional[torch.Tensor] = None, xq_out: Optional[torch.Tensor] = None,
                  sx_out: Optional[torch.Tensor] = None, splits: int = 0, ws: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """y = acc * w_scale[n] * s_x with x fp16 [K] quantised per token in the
    kernel (s_x = max|x| / 127, xq = clamp(rint(x / s_x), +-127)); acc int32."""
    N, K = Wq.shape
    if y is None:
        y = torch.empty(N, dtype=torch.float32, device=Wq.device)
    if ws is None:
        ws = workspace(W8A8_DYN, 1, N, K, splits, Wq.device)
    wp, wn = _ws(ws)
    opt = lambda t, dt, name, shape: _dev(t, dt, name, shape) if t is not None else None  # noqa: E731
    _check(lib().gemv_w8a8_dyn(_dev(Wq, torch.int8, "Wq"), _dev(w_scale, torch.float32, "w_scale", (N,)),
                               _dev(x, torch.float16, "x", (K,)), _dev(y, torch.float32, "y", (N,)),
                               opt(acc_out, torch.int32, "acc_out", (N,)), opt(xq_out, torch.int8, "xq_out", (K,)),
                               opt(sx_out, torch.float32, "sx_out", (1,)), N, K, splits, wp, wn, _stream(stream)),
           "gemv_w8a8_dyn")
    return y


def packed_w4_bytes(N: int, K: int, group: int = 128) -> Tuple[int, int]:
    return int(lib().wsg_w4_packed_weight_bytes(N, K)), int(lib().wsg_w4_packed_scale_bytes(N, K, group))


def pack_w4(Wc: torch.Tensor, s4: torch.Tensor, group: int = 128, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Load-time packing of canonical int4 words Wc int32/uint32 [N, K/8] and
    fp16 scales s4 [N, K/group] into the kernels' tile layout."""
    N, K8 = Wc.shape
    K = K8 * 8
    if Wc.dtype not in (torch.int32, torch.uint32):
        raise TypeError("Wc must hold 32-bit words (int32 or uint32)")
    wb, sb = packed_w4_bytes(N, K, group)
    Wp = torch.empty(max(wb, 16), dtype=torch.uint8, device=Wc.device)
    Sp = torch.empty(max(sb, 16), dtype=torch.uint8, device=Wc.device)
    _check(lib().wsg_pack_w4(_dev(Wc, Wc.dtype, "Wc"), _dev(s4, torch.float16, "s4", (N, K // group)),
                             Wp.data_ptr(), Sp.data_ptr(), N, K, group, _stream(stream)), "wsg_pack_w4")
    return Wp, Sp


def gemv_w4a16(Wp: torch.Tensor, Sp: torch.Tensor, x: torch.Tensor, N: int, group: int = 128,
               y: Optional[torch.Tensor] = None, splits: int = 0, ws: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    """y[m,n] = sum_k (q[n,k]-8) s4[n,k/128] x[m,k]; x fp16 [M,K] or [K]; y fp32 [M,N] (or [N])."""
    squeeze = x.dim() == 1
    X = x.reshape(1, -1) if squeeze else x
    M, K = X.shape
    if y is None:
        y = torch.empty((M, N) if not squeeze else (N,), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(W4A16, M, N, K, splits, x.device)
    wp, wn = _ws(ws)
    wb, sb = packed_w4_bytes(N, K, group)
    if Wp.numel() * Wp.element_size() < wb or Sp.numel() * Sp.element_size() < sb:
        raise ValueError("packed buffers are smaller than this (N, K) needs")
    _check(lib().gemv_w4a16(_dev(Wp, Wp.dtype, "Wp"), _dev(Sp, Sp.dtype, "Sp"), _dev(X, torch.float16, "x"),
                            _dev(y, torch.float32, "y"), M, N, K, group, splits, wp, wn, _stream(stream)),
           "gemv_w4a16")
    return y


def gemv_w4a8(Wp: torch.Tensor, Sp: torch.Tensor, x: torch.Tensor, N: int, group: int = 128,
              y: Optional[torch.Tensor] = None, xq_out: Optional[torch.Tensor] = None,
              sx_out: Optional[torch.Tensor] = None, splits: int = 0, ws: Optional[torch.Tensor] = None,
              stream=None) -> torch.Tensor:
    """y[n] = s_x sum_k (q[n,k]-8) s4[n,k/128] xq[k], with x fp16 [K] quantised to int8 per token
    inside the kernel; optional xq_out int8 [K] and sx_out fp32 [1] receive the codes and scale."""
    K = x.shape[0]
    if y is None:
        y = torch.empty(N, dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(W4A8, 1, N, K, splits, x.device)
    wp, wn = _ws(ws)
    wb, sb = packed_w4_bytes(N, K, group)
    if Wp.numel() * Wp.element_size() < wb or Sp.numel() * Sp.element_size() < sb:
        raise ValueError("packed buffers are smaller than this (N, K) needs")
    xq_p = _dev(xq_out, torch.int8, "xq_out", (K,)) if xq_out is not None else None
    sx_p = _dev(sx_out, torch.float32, "sx_out", (1,)) if sx_out is not None else None
    _check(lib().gemv_w4a8(_dev(Wp, Wp.dtype, "Wp"), _dev(Sp, Sp.dtype, "Sp"), _dev(x, torch.float16, "x", (K,)),
                           _dev(y, torch.float32, "y", (N,)), xq_p, sx_p, N, K, group, splits, wp, wn,
                           _stream(stream)), "gemv_w4a8")
    return y


def read_probe(buf: torch.Tensor, out: torch.Tensor, grid: int = 0, stream=None) -> None:
    _check(lib().wsg_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(),
                                _dev(out, torch.float32, "out"), grid, _stream(stream)), "wsg_read_probe")


def tune_set(key: str, value: int) -> None:
    """Launch-table override for tuning sweeps (value < 0 restores the default)."""
    _check(lib().wsg_tune_set(key.encode(), int(value)), f"wsg_tune_set({key})")


def read_probe_grid(nbytes: int) -> int:
    return int(lib().wsg_read_probe_grid(nbytes))


class Linear:
    """Description of one linear of a decode step (all tensors on the GPU)."""

    def __init__(self, kind: int, W: torch.Tensor, x: torch.Tensor, y: torch.Tensor, N: int, K: int, M: int = 1,
                 scale: Optional[torch.Tensor] = None, x_scale: Optional[torch.Tensor] = None,
                 acc_out: Optional[torch.Tensor] = None, group: int = 0, splits: int = 0,
                 argmax_idx: Optional[torch.Tensor] = None, argmax_val: Optional[torch.Tensor] = None,
                 conv_w: Optional[torch.Tensor] = None, conv_bias: Optional[torch.Tensor] = None,
                 conv_state: Optional[torch.Tensor] = None, conv_out: Optional[torch.Tensor] = None,
                 conv_silu: bool = False, y16: Optional[torch.Tensor] = None):
        self.kind, self.W, self.x, self.y, self.N, self.K, self.M = kind, W, x, y, N, K, M
        self.scale, self.x_scale, self.acc_out, self.group, self.splits = scale, x_scale, acc_out, group, splits
        self.argmax_idx, self.argmax_val = argmax_idx, argmax_val
        self.conv_w, self.conv_bias, self.conv_state, self.conv_out = conv_w, conv_bias, conv_state, conv_out
        self.conv_width = 0 if conv_w is None or conv_w.dim() != 2 else int(conv_w.shape[1])
        self.conv_silu = int(bool(conv_silu))
        self.y16 = y16   # optional fp16 copy of y, rounded to nearest even
        self._check()

    def _check(self) -> None:
        """Every tensor against the sizes given beside it, before the plan
        freezes their addresses: a mis-sized buffer would otherwise become an
        out-of-bounds load or store inside a kernel."""
        f16, i8, f32, i32 = (torch.float16,), (torch.int8,), (torch.float32,), (torch.int32,)
        anyd = (torch.uint8, torch.int8, torch.int16, torch.int32, torch.uint32, torch.int64, torch.float16,
                torch.float32)
        M, N, K, kind = self.M, self.N, self.K, self.kind
        req = []  # (tensor, dtypes, name, numel, min_bytes, optional)
        req.append((self.y, f32, "y", M * N, None, False))
        if kind == F16:
            req += [(self.W, f16, "W", N * K, None, False), (self.x, f16, "x", M * K, None, False)]
        elif kind in (W8A8, W8A8_DYN):
            req += [(self.W, i8, "W", N * K, None, False),
                    (self.x, i8 if kind == W8A8 else f16, "x", K, None, False),
                    (self.scale, f32, "scale", N, None, True), (self.x_scale, f32, "x_scale", 1, None, True),
                    (self.acc_out, i32, "acc_out", N, None, True)]
        elif kind in (W4A16, W4A8):
            wb, sb = packed_w4_bytes(N, K, self.group) if self.group > 0 else (0, 0)
            req += [(self.W, anyd, "W (packed)", None, wb, False), (self.scale, anyd, "scale (packed)", None, sb, True),
                    (self.x, f16, "x", M * K, None, False)]
        req += [(self.argmax_idx, i32, "argmax_idx", M, None, True), (self.argmax_val, f32, "argmax_val", M, None, True)]
        if self.conv_w is not None:
            Wc = self.conv_width
            req += [(self.conv_w, f16, "conv_w", N * Wc, None, False), (self.conv_bias, f32, "conv_bias", N, None, True),
                    (self.conv_state, f32, "conv_state", N * max(Wc - 1, 0), None, False),
                    (self.conv_out, f32, "conv_out", N, None, False)]
        req.append((self.y16, f16, "y16", None, 2 * M * N, True))
        # sizes of every tensor first, then where they live
        for t, dt, name, numel, mb, opt in req:
            _check_tensor(t, dt, name, numel=numel, min_bytes=mb, optional=opt, device=False)
        for t, dt, name, numel, mb, opt in req:
            _check_tensor(t, dt, name, numel=numel, min_bytes=mb, optional=opt)

    def c(self) -> wsg_linear:
        p = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
        return wsg_linear(self.kind, self.M, self.N, self.K, p(self.W), p(self.scale), p(self.x), p(self.x_scale),
                          p(self.y), p(self.acc_out), self.group, self.splits, p(self.argmax_idx),
                          p(self.argmax_val), p(self.conv_w), p(self.conv_bias), p(self.conv_state),
                          p(self.conv_out), self.conv_width, self.conv_silu, p(self.y16))


class DecodeStep:
    """A captured decode step (wsg_decode_step_create / decode_step_linears).

    The tensors of every Linear are kept referenced for the plan's life,
    because the plan holds their device addresses."""

    def __init__(self, linears: Sequence[Linear], mode: int = STEP_GROUPED, stream=None):
        self._keep = list(linears)
        arr = (wsg_linear * max(1, len(linears)))(*[l.c() for l in linears])
        h = ctypes.c_void_p()
        _check(lib().wsg_decode_step_create(arr, len(linears), mode, _stream(stream), ctypes.byref(h)),
               "wsg_decode_step_create")
        self._h = h
        self.mode = mode

    def __call__(self, stream=None) -> None:
        if self._h is None:
            raise WsgError(8, "decode_step_linears", "destroyed plan")
        _check(lib().decode_step_linears(self._h, _stream(stream)), "decode_step_linears")

    def info(self) -> Tuple[int, int]:
        a, b = ctypes.c_int32(), ctypes.c_int64()
        _check(lib().wsg_decode_step_info(self._h, ctypes.byref(a), ctypes.byref(b), None), "wsg_decode_step_info")
        return a.value, b.value

    def give_ups(self, stream=None) -> int:
        """Waits of a persistent plan that gave up since the last call (synchronises the stream)."""
        g = ctypes.c_uint32()
        _check(lib().wsg_decode_step_status(self._h, _stream(stream), ctypes.byref(g)), "wsg_decode_step_status")
        return int(g.value)

    def set_trace(self, buf: Optional[torch.Tensor]) -> None:
        """Per-unit timestamps of a persistent plan into `buf` (int64 on the
        device, at least 4 words per work unit) for every later step; None
        stops tracing (wsg_decode_step_trace).  The buffer is kept referenced
        while it is set."""
        if buf is None:
            _check(lib().wsg_decode_step_trace(self._h, None, 0), "wsg_decode_step_trace")
            self._trace = None
            return
        if buf.dtype != torch.int64 or not buf.is_cuda or not buf.is_contiguous():
            raise ValueError("trace buffer: a contiguous int64 tensor on the device")
        _check(lib().wsg_decode_step_trace(self._h, buf.data_ptr(), buf.numel()), "wsg_decode_step_trace")
        self._trace = buf

    def uses_graph(self) -> bool:
        g = ctypes.c_int32()
        _check(lib().wsg_decode_step_info(self._h, None, None, ctypes.byref(g)), "wsg_decode_step_info")
        return bool(g.value)

    def close(self) -> None:
        if self._h is not None:
            _check(lib().wsg_decode_step_destroy(self._h), "wsg_decode_step_destroy")
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
