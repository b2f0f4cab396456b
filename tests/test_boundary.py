"""The C-ABI boundary on the CPU: the library loads, exports every function
include/wsgemv.h declares, and rejects bad arguments before any HIP call.

Pointers here are fake device addresses that are never dereferenced: every
call below fails validation, which happens before anything is launched.
"""
import ctypes

import pytest

from weight_streaming_gemv_decode_amd import wsgemv

FAKE = 0x7F0000000000          # 256-byte aligned, never dereferenced
MIS = FAKE + 2                 # misaligned
OK, NULL, SHAPE, ALIGN, UNSUP, WS, HIP, NOMEM, STATE = range(9)


def split_ws(S, N, tile_rows, dyn=False):
    """Workspace of a split fp16/int8 linear: S rows of 4-byte partials (and
    for W8A8_DYN 256 bytes for the published scale), then, from the next
    256-byte boundary, one 4-byte arrival counter per row tile."""
    part = S * N * 4 + (256 if dyn else 0)
    return (part + 255) // 256 * 256 + (N + tile_rows - 1) // tile_rows * 4


@pytest.fixture(scope="module")
def L():
    return wsgemv.lib()


def test_exports_every_declared_function(L):
    names = wsgemv.header_functions()
    assert {"gemv_f16", "gemv_w8a8", "gemv_w4a16", "gemv_w4a8", "decode_step_linears", "wsg_pack_w4",
            "gemv_f16_argmax", "wsg_argmax_f32", "causal_conv1d_step", "wsg_topk_f32", "wsg_topk_ws_bytes",
            "wsg_decode_step_create"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/wsgemv.h but not exported"


def test_status_strings(L):
    for s in range(9):
        assert L.wsg_status_string(s)
    assert L.wsg_status_string(0) == b"ok"
    assert b"gfx950" in L.wsg_build_info()


def test_gemv_f16_validation(L):
    f = L.gemv_f16
    assert f(FAKE, FAKE, FAKE, -1, 64, 0, None, 0, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, 4, 12, 0, None, 0, None) == SHAPE          # K % 8
    assert f(None, FAKE, FAKE, 4, 64, 0, None, 0, None) == NULL
    assert f(FAKE, None, FAKE, 4, 64, 0, None, 0, None) == NULL
    assert f(FAKE, FAKE, None, 4, 64, 0, None, 0, None) == NULL
    assert f(MIS, FAKE, FAKE, 4, 64, 0, None, 0, None) == ALIGN
    assert f(FAKE, MIS, FAKE, 4, 64, 0, None, 0, None) == ALIGN
    assert f(FAKE, FAKE, FAKE + 1, 4, 64, 0, None, 0, None) == ALIGN
    assert f(FAKE, FAKE, FAKE, 4, 64, -1, None, 0, None) == SHAPE          # negative split
    assert f(FAKE, FAKE, FAKE, 4, 64, 9, None, 0, None) == SHAPE           # more slices than vectors
    assert f(FAKE, FAKE, FAKE, 4, 1024, 2, None, 0, None) == WS            # split needs workspace
    need = L.wsg_workspace_bytes(0, 1, 4, 1024, 2)
    assert need == split_ws(2, 4, 32)
    assert f(FAKE, FAKE, FAKE, 4, 1024, 2, FAKE, need - 1, None) == WS
    assert f(FAKE, FAKE, FAKE, 4, 1024, 2, FAKE + 16, need, None) == ALIGN
    assert f(None, None, None, 0, 64, 0, None, 0, None) == OK               # N = 0: no-op, nothing launched


def test_gemv_f16_static_validation(L):
    f = L.gemv_f16_static
    assert f(FAKE, FAKE, FAKE, -1, 64, 0, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, 4, 12, 0, None) == SHAPE                   # K % 8
    assert f(None, FAKE, FAKE, 4, 64, 0, None) == NULL
    assert f(FAKE, FAKE, FAKE + 1, 4, 64, 0, None) == ALIGN
    assert f(FAKE, FAKE, FAKE, 4, 64, 9, None) == SHAPE                   # more slices than vectors
    # partials beyond the library's scratch array are refused before any HIP call
    cap = wsgemv.STATIC_SCRATCH_BYTES
    N = cap // 8 + 1
    assert f(FAKE, FAKE, FAKE, N, 4096, 2, None) == WS
    assert f(None, None, None, 0, 64, 0, None) == OK                      # N = 0: no-op


def test_gemv_w8a8_validation(L):
    f = L.gemv_w8a8
    args = lambda **kw: [kw.get("W", FAKE), kw.get("ws_", FAKE), kw.get("x", FAKE), kw.get("xs", FAKE),  # noqa
                         kw.get("y", FAKE), kw.get("acc", None), kw.get("N", 8), kw.get("K", 64),
                         kw.get("S", 0), None, 0, None]
    assert f(*args(K=24)) == SHAPE                                          # K % 16
    assert f(*args(W=None)) == NULL
    assert f(*args(ws_=None)) == NULL
    assert f(*args(xs=None)) == NULL
    assert f(*args(acc=FAKE + 2)) == ALIGN
    assert f(*args(x=MIS)) == ALIGN
    assert f(*args(N=-3)) == SHAPE


def test_w4_validation_and_sizes(L):
    assert L.wsg_w4_packed_weight_bytes(17, 256) == 32 * 128                 # rows padded to 16
    assert L.wsg_w4_packed_scale_bytes(17, 256, 128) == 32 * 4 * 2          # 4 scales per (row, quad)
    assert L.wsg_w4_packed_weight_bytes(16, 100) == 0
    assert L.wsg_pack_w4(FAKE, FAKE, FAKE, FAKE, 16, 256, 64, None) == UNSUP
    assert L.wsg_pack_w4(FAKE, FAKE, FAKE, FAKE, 16, 200, 128, None) == SHAPE
    assert L.wsg_pack_w4(None, FAKE, FAKE, FAKE, 16, 256, 128, None) == NULL
    assert L.wsg_pack_w4(FAKE, FAKE, MIS, FAKE, 16, 256, 128, None) == ALIGN
    f = L.gemv_w4a16
    assert f(FAKE, FAKE, FAKE, FAKE, 9, 16, 256, 128, 0, None, 0, None) == UNSUP    # M > 8
    assert f(FAKE, FAKE, FAKE, FAKE, 0, 16, 256, 128, 0, None, 0, None) == SHAPE    # M = 0
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 16, 256, 64, 0, None, 0, None) == UNSUP     # group
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 16, 192, 128, 0, None, 0, None) == SHAPE    # K % 128
    assert f(FAKE, None, FAKE, FAKE, 1, 16, 256, 128, 0, None, 0, None) == NULL
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 16, 256, 128, 3, None, 0, None) == SHAPE    # slice past K
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 16, 1024, 128, 2, None, 0, None) == WS
    g = L.gemv_w4a8
    a8 = lambda **kw: [kw.get("Wp", FAKE), FAKE, kw.get("x", FAKE), FAKE, kw.get("xq", None),  # noqa: E731
                       kw.get("sx", None), kw.get("N", 16), kw.get("K", 256), kw.get("group", 128),
                       kw.get("S", 0), None, 0, None]
    assert g(*a8(group=64)) == UNSUP
    assert g(*a8(K=192)) == SHAPE                                               # K % 128
    assert g(*a8(Wp=None)) == NULL
    assert g(*a8(x=MIS)) == ALIGN
    assert g(*a8(xq=FAKE + 4)) == ALIGN                                         # codes 8-byte aligned
    assert g(*a8(sx=FAKE + 2)) == ALIGN
    assert g(*a8(S=3)) == SHAPE                                                 # slice past K
    assert g(*a8(N=16, K=1024, S=2)) == WS
    # 2 x 16 partials, then one counter (16 rows: a single 16-row tile)
    assert L.wsg_workspace_bytes(3, 1, 16, 1024, 2) == 256 + 4
    assert g(*a8(N=0)) == OK                                                    # nothing to do


def test_argmax_validation(L):
    g = L.wsg_argmax_f32
    assert g(FAKE, 0, FAKE, None, FAKE, 256, None) == SHAPE                    # no values
    assert g(FAKE, 1 << 31, FAKE, None, FAKE, 256, None) == UNSUP             # index must fit int32
    assert g(FAKE, 10, None, None, FAKE, 256, None) == NULL                   # token required
    assert g(None, 10, FAKE, None, FAKE, 256, None) == NULL
    assert g(FAKE + 2, 10, FAKE, None, FAKE, 256, None) == ALIGN
    assert g(FAKE, 10, FAKE + 1, None, FAKE, 256, None) == ALIGN
    assert g(FAKE, 10, FAKE, FAKE + 2, FAKE, 256, None) == ALIGN
    assert g(FAKE, 10, FAKE, None, FAKE, 255, None) == WS
    assert g(FAKE, 10, FAKE, None, None, 0, None) == WS
    assert g(FAKE, 10, FAKE, None, FAKE + 8, 256, None) == ALIGN
    f = L.gemv_f16_argmax
    assert f(FAKE, FAKE, FAKE, FAKE, None, 0, 64, 0, FAKE, 256, None) == SHAPE   # N = 0: no token
    assert f(FAKE, FAKE, FAKE, None, None, 4, 64, 0, FAKE, 256, None) == NULL
    assert f(FAKE, FAKE, FAKE, FAKE, None, 4, 60, 0, FAKE, 256, None) == SHAPE   # K % 8
    assert f(FAKE, FAKE, FAKE, FAKE, None, 4, 64, 0, FAKE, 128, None) == WS
    need = L.wsg_workspace_bytes(0 | 0x100, 1, 4, 1024, 2)
    assert need == 256 + split_ws(2, 4, 32)                                   # one key, then the split
    assert f(FAKE, FAKE, FAKE, FAKE, None, 4, 1024, 2, FAKE, need - 1, None) == WS
    assert L.wsg_workspace_bytes(2 | 0x100, 1, 16, 256, 0) == 0                  # int4: no fused token
    out = ctypes.c_void_p()
    lin = lambda kind, tok, val=None, N=64: wsgemv.wsg_linear(kind, 1, N, 256, FAKE, FAKE, FAKE, FAKE,  # noqa
                                                             FAKE, None, 128 if kind >= 2 else 0, 0, tok, val)
    for kind, tok, val, N, want in ((2, FAKE, None, 1 << 31, UNSUP), (0, FAKE + 2, None, 64, ALIGN),
                                    (0, None, FAKE, 64, NULL), (0, FAKE, None, 1 << 31, UNSUP)):
        arr = (wsgemv.wsg_linear * 1)(lin(kind, tok, val, N))
        assert L.wsg_decode_step_create(arr, 1, 0, None, ctypes.byref(out)) == want, (kind, want)


def test_conv1d_validation(L):
    f = L.causal_conv1d_step
    assert f(FAKE, FAKE, None, FAKE, FAKE, -1, 4, 0, None) == SHAPE
    assert f(FAKE, FAKE, None, FAKE, FAKE, 10, 1, 0, None) == UNSUP             # W = 2..8
    assert f(FAKE, FAKE, None, FAKE, FAKE, 10, 9, 0, None) == UNSUP
    assert f(None, FAKE, None, FAKE, FAKE, 10, 4, 0, None) == NULL
    assert f(FAKE, None, None, FAKE, FAKE, 10, 4, 0, None) == NULL
    assert f(FAKE, FAKE, None, None, FAKE, 10, 4, 0, None) == NULL
    assert f(FAKE, FAKE, None, FAKE, None, 10, 4, 0, None) == NULL
    assert f(FAKE, FAKE + 1, None, FAKE, FAKE, 10, 4, 0, None) == ALIGN
    assert f(FAKE, FAKE, FAKE + 2, FAKE, FAKE, 10, 4, 0, None) == ALIGN
    assert f(None, FAKE, None, FAKE, FAKE, 0, 4, 0, None) == OK                 # no channels
    out = ctypes.c_void_p()
    for kind, M, width, want in ((2, 4, 4, UNSUP), (3, 2, 4, UNSUP), (0, 1, 9, UNSUP), (0, 1, 4, OK), (2, 1, 4, OK),
                                 (3, 1, 4, OK)):
        l = wsgemv.wsg_linear(kind, M, 64, 256, FAKE, FAKE if kind >= 2 else None, FAKE, None, FAKE, None,
                              128 if kind >= 2 else 0, 0, None, None, FAKE, None, FAKE, FAKE, width, 0)
        arr = (wsgemv.wsg_linear * 1)(l)
        got = L.wsg_decode_step_create(arr, 1, 0x100, None, ctypes.byref(out)) if want != OK else \
            _validate_only(L, arr)
        assert got == want, (kind, width, got)


def _validate_only(L, arr):
    # a valid descriptor would allocate and launch: check only that every
    # rejection path above is specific, by breaking one field at a time
    bad = wsgemv.wsg_linear.from_buffer_copy(arr[0])
    bad.conv_state = None
    return OK if L.wsg_decode_step_create((wsgemv.wsg_linear * 1)(bad), 1, 0x100, None,
                                          ctypes.byref(ctypes.c_void_p())) == NULL else -1


def test_topk_validation(L):
    f = L.wsg_topk_f32
    need = L.wsg_topk_ws_bytes(1000, 8)
    assert need > 0 and need % 256 == 0
    assert L.wsg_topk_ws_bytes(1000, 0) == 0 and L.wsg_topk_ws_bytes(1000, 65) == 0 and L.wsg_topk_ws_bytes(5, 8) == 0
    assert f(FAKE, 1000, 0, FAKE, None, FAKE, need, None) == SHAPE             # k >= 1
    assert f(FAKE, 5, 8, FAKE, None, FAKE, need, None) == SHAPE                # k <= N
    assert f(FAKE, 1000, 65, FAKE, None, FAKE, need, None) == UNSUP            # k <= 64
    assert f(FAKE, 0, 1, FAKE, None, FAKE, need, None) == SHAPE
    assert f(None, 1000, 8, FAKE, None, FAKE, need, None) == NULL
    assert f(FAKE, 1000, 8, None, None, FAKE, need, None) == NULL
    assert f(FAKE + 2, 1000, 8, FAKE, None, FAKE, need, None) == ALIGN
    assert f(FAKE, 1000, 8, FAKE, None, FAKE, need - 1, None) == WS
    assert f(FAKE, 1000, 8, FAKE, None, FAKE + 16, need, None) == ALIGN


def test_launch_table(L):
    # The table is a pure host function of the shape.
    assert L.wsg_plan_splits(0, 1, 248320, 1024) >= 1
    assert L.wsg_plan_splits(0, 1, 64, 32768) >= 2       # slice must fit the LDS activation stage
    assert L.wsg_plan_splits(0, 1, 16, 8192) > 1         # very few rows: split k
    assert L.wsg_plan_splits(1, 1, 4096, 14336) == 1     # enough rows: no split
    assert L.wsg_plan_splits(0, 1, 248320, 1024) * 248320 * 4 == L.wsg_workspace_bytes(0, 1, 248320, 1024, 0) \
        or L.wsg_plan_splits(0, 1, 248320, 1024) == 1
    # 2048x2048 fp16 (256 vectors a row): slices of 128 and 86 vectors take
    # 8-row tiles, slices of 64 vectors 32-row tiles
    for S, rows in ((2, 8), (3, 8), (4, 32)):
        assert L.wsg_workspace_bytes(0, 1, 2048, 2048, S) == split_ws(S, 2048, rows)
    assert L.wsg_workspace_bytes(0, 1, 2048, 2048, 1) == 0
    assert L.wsg_workspace_bytes(0, 1, 248320, 1024, 2) == split_ws(2, 248320, 32)


def test_decode_step_validation(L):
    out = ctypes.c_void_p()
    lin = wsgemv.wsg_linear(0, 1, 64, 64, FAKE, None, FAKE, None, FAKE, None, 0, 0)
    arr = (wsgemv.wsg_linear * 1)(lin)
    assert L.wsg_decode_step_create(arr, 1, 7, None, ctypes.byref(out)) == UNSUP   # bad mode
    assert L.wsg_decode_step_create(arr, 1, 0x300, None, ctypes.byref(out)) == UNSUP  # eager and forced graph
    assert L.wsg_decode_step_create(arr, 1, 0x400, None, ctypes.byref(out)) == UNSUP  # unknown flag
    assert L.wsg_decode_step_create(arr, -1, 0, None, ctypes.byref(out)) == SHAPE
    assert L.wsg_decode_step_create(None, 1, 0, None, ctypes.byref(out)) == NULL
    assert L.wsg_decode_step_create(arr, 1, 0, None, None) == NULL
    bad = (wsgemv.wsg_linear * 1)(wsgemv.wsg_linear(0, 2, 64, 64, FAKE, None, FAKE, None, FAKE, None, 0, 0))
    assert L.wsg_decode_step_create(bad, 1, 0, None, ctypes.byref(out)) == UNSUP   # fp16 with M = 2
    bad = (wsgemv.wsg_linear * 1)(wsgemv.wsg_linear(5, 1, 64, 64, FAKE, None, FAKE, None, FAKE, None, 0, 0))
    assert L.wsg_decode_step_create(bad, 1, 0, None, ctypes.byref(out)) == UNSUP   # unknown kind
    bad = (wsgemv.wsg_linear * 1)(wsgemv.wsg_linear(1, 1, 64, 64, FAKE, None, FAKE, FAKE, FAKE, None, 0, 0))
    assert L.wsg_decode_step_create(bad, 1, 0, None, ctypes.byref(out)) == NULL    # W8A8 without scales
    bad = (wsgemv.wsg_linear * 1)(wsgemv.wsg_linear(0, 1, 64, 4096, FAKE, None, FAKE, None, FAKE, None, 0, 2))
    assert L.wsg_decode_step_create(bad, 1, 1, None, ctypes.byref(out)) == UNSUP   # GROUPED forbids splits
    bad = (wsgemv.wsg_linear * 1)(wsgemv.wsg_linear(3, 2, 64, 256, FAKE, FAKE, FAKE, None, FAKE, None, 128, 0))
    assert L.wsg_decode_step_create(bad, 1, 0, None, ctypes.byref(out)) == UNSUP   # W4A8 with M = 2
    assert L.decode_step_linears(None, None) == STATE
    assert L.wsg_decode_step_destroy(None) == STATE


def test_binding_rejects_cpu_tensors():
    import torch
    W = torch.zeros(4, 16, dtype=torch.float16)
    x = torch.zeros(16, dtype=torch.float16)
    with pytest.raises(ValueError):
        wsgemv.gemv_f16(W, x, y=torch.zeros(4), splits=1)


def test_tuning_overrides_validated():
    keys = ("dense_R", "dense_CH", "w4_B")
    try:
        with pytest.raises(wsgemv.WsgError):
            wsgemv.tune_set("no_such_key", 1)
        wsgemv.tune_set("dense_R", 3)          # alone it is only recorded
        with pytest.raises(wsgemv.WsgError):
            wsgemv.tune_set("dense_CH", 2)     # (R=3, CH=2) is not a built kernel shape
        with pytest.raises(wsgemv.WsgError):
            wsgemv.tune_set("w4_B", 6)
        wsgemv.tune_set("dense_R", 8)
        wsgemv.tune_set("dense_CH", 1)
    finally:
        for k in keys:
            wsgemv.tune_set(k, -1)


def test_y16_validation(L):
    """A linear's fp16 output copy: 2-byte aligned; a GROUPED plan rejects a
    list in which one linear's x overlaps a y16 (the units run in no fixed
    order), before any HIP call."""
    out = ctypes.c_void_p()
    y16 = FAKE + 0x100000                       # a.y16 spans 64 rows x 2 bytes = 128 bytes
    a = wsgemv.wsg_linear(0, 1, 64, 64, FAKE, None, FAKE, None, FAKE + 0x10000, None, 0, 0)
    a.y16 = y16 + 1
    assert L.wsg_decode_step_create((wsgemv.wsg_linear * 1)(a), 1, 1, None, ctypes.byref(out)) == ALIGN
    a.y16 = y16
    # an int4 linear whose fp16 x (128 values, 256 bytes) starts inside, at, or ends inside a.y16
    for x_at in (y16, y16 + 64, y16 + 112, y16 - 240):
        b = wsgemv.wsg_linear(2, 1, 64, 128, FAKE, FAKE, x_at, None, FAKE + 0x20000, None, 128, 0)
        got = L.wsg_decode_step_create((wsgemv.wsg_linear * 2)(a, b), 2, 1, None, ctypes.byref(out))
        assert got == UNSUP, (hex(x_at), got)
    # a W8A8 linear's int8 x is K bytes: 80 bytes from y16 - 64 reach into a.y16
    c = wsgemv.wsg_linear(1, 1, 64, 80, FAKE, FAKE, y16 - 64, FAKE, FAKE + 0x30000, None, 0, 0)
    assert L.wsg_decode_step_create((wsgemv.wsg_linear * 2)(c, a), 2, 1, None, ctypes.byref(out)) == UNSUP


def test_w8a8_dyn_validation(L):
    """int8 weights with fp16 activations quantised in the kernel: every
    rejection returns before any HIP call."""
    f = L.gemv_w8a8_dyn
    args = lambda **kw: [kw.get(k, v) for k, v in (("Wq", FAKE), ("sw", FAKE), ("x", FAKE), ("y", FAKE),  # noqa: E731
                                                  ("acc", None), ("xq", None), ("sx", None), ("N", 64),
                                                  ("K", 128), ("S", 0), ("ws", None), ("wsb", 0), ("st", None))]
    assert f(*args(K=100)) == SHAPE                   # K % 16
    assert f(*args(N=-1)) == SHAPE
    assert f(*args(Wq=None)) == NULL
    assert f(*args(x=None)) == NULL
    assert f(*args(y=None)) == NULL
    assert f(*args(sw=None)) == NULL
    assert f(*args(x=MIS)) == ALIGN
    assert f(*args(acc=FAKE + 2)) == ALIGN
    assert f(*args(xq=FAKE + 8)) == ALIGN             # codes are written 16 bytes at a time
    assert f(*args(sx=FAKE + 2)) == ALIGN
    assert f(*args(sw=FAKE + 2)) == ALIGN
    assert f(*args(S=200)) == SHAPE                   # more slices than 16-byte vectors
    assert f(*args(N=0)) == OK                        # nothing to do
    # split partials, 256 bytes for the activation scale the first work unit
    # publishes, then the counters (448-vector slices: 32-row tiles)
    assert L.wsg_workspace_bytes(4, 1, 4096, 14336, 2) == split_ws(2, 4096, 32, dyn=True)
    assert L.wsg_workspace_bytes(4, 1, 4096, 14336, 1) == 0
    assert L.wsg_plan_splits(4, 1, 4096, 14336) == L.wsg_plan_splits(1, 1, 4096, 14336)
    # in a decode step: M = 1 only, and the activation scale is computed, not given
    out = ctypes.c_void_p()
    for M, xs, want in ((2, None, UNSUP), (1, FAKE, UNSUP), (1, None, NULL)):
        lin = wsgemv.wsg_linear(4, M, 64, 128, FAKE, None if want == NULL else FAKE, FAKE, xs, FAKE, None, 0, 0)
        got = L.wsg_decode_step_create((wsgemv.wsg_linear * 1)(lin), 1, 1, None, ctypes.byref(out))
        assert got == want, (M, xs, got)


def test_launch_size_limits(L):
    """Shapes whose launches would exceed HIP's 32-bit work-item count are
    rejected before any size is narrowed or any kernel is launched; the
    largest accepted ones still pass validation (checked with a NULL output,
    so nothing is launched)."""
    big = 1 << 33                      # rows: N / 4 units would not fit a launch
    assert L.gemv_f16(FAKE, FAKE, FAKE, big, 64, 0, None, 0, None) == UNSUP
    assert L.gemv_f16(FAKE, FAKE, FAKE, big, 0, 0, None, 0, None) == UNSUP       # K = 0 zero-fill launch too
    assert L.gemv_f16(FAKE, FAKE, FAKE, 1 << 26, 4096, 16, FAKE, 1 << 40, None) == UNSUP  # forced splits
    assert L.gemv_f16(FAKE, FAKE, None, 1 << 24, 64, 0, None, 0, None) == NULL   # 16M rows: fits
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, None, big, 64, 0, None, 0, None]
    assert L.gemv_w8a8(*args) == UNSUP
    assert L.gemv_w4a16(FAKE, FAKE, FAKE, FAKE, 8, big // 8, 256, 128, 0, None, 0, None) == UNSUP
    assert L.gemv_w4a16(FAKE, FAKE, FAKE, None, 1, 1 << 24, 256, 128, 0, None, 0, None) == NULL
    assert L.wsg_pack_w4(FAKE, FAKE, FAKE, FAKE, big, 1 << 14, 128, None) == UNSUP
    assert L.causal_conv1d_step(FAKE, FAKE, None, FAKE, FAKE, 1 << 40, 4, 0, None) == UNSUP


def test_chain_grid_sizing(L):
    """The persistent launch's grid: never more workgroups than units, nor
    than can be resident at once (blocks per CU from the occupancy query,
    optionally capped), and 0 for empty or invalid counts."""
    g = L.wsg_chain_grid
    assert g(10**9, 5, 256, 4) == 4 * 256      # capped below the resident count
    assert g(10**9, 3, 256, 4) == 3 * 256      # the resident count is the limit
    assert g(10**9, 5, 256, 0) == 5 * 256      # no cap
    assert g(100, 5, 256, 4) == 100            # fewer units than slots
    assert g(0, 5, 256, 4) == 0 and g(10, 0, 256, 4) == 0 and g(10, 5, 0, 4) == 0 and g(-1, 5, 256, 4) == 0
    for units in (1, 255, 256, 1023, 1024, 1025, 36864):
        for per in (1, 2, 5, 8):
            for cap in (-1, 0, 1, 4, 16):
                G = g(units, per, 256, cap)
                assert 1 <= G <= units and G <= per * 256 and (cap <= 0 or G <= cap * 256)


def test_persistent_validation(L):
    """WSG_STEP_PERSISTENT accepts only fp16 M = 1 lists whose inputs are
    plain buffers or lie wholly inside one earlier linear's y16; every
    rejection returns before any HIP call."""
    out = ctypes.c_void_p()
    P = 2
    y16 = FAKE + 0x100000                       # 64 outputs x 2 bytes

    def lin(kind=0, N=64, K=64, x=FAKE, y=None, y16_=None, M=1, splits=0, **kw):
        a = wsgemv.wsg_linear(kind, M, N, K, FAKE, kw.get("scale"), x, kw.get("xs"), y or FAKE + 0x10000 * (1 + N % 7),
                              None, kw.get("group", 0), splits)
        a.y16 = y16_
        for k in ("argmax_idx",):
            if k in kw:
                setattr(a, k, kw[k])
        return a

    def create(*ls, mode=P):
        return L.wsg_decode_step_create((wsgemv.wsg_linear * len(ls))(*ls), len(ls), mode, None, ctypes.byref(out))

    a = lin(N=64, K=64, y=FAKE + 0x10000, y16_=y16)
    assert create(a, mode=P | 0x100) == UNSUP                                     # no graph flags
    assert create(a, mode=P | 0x200) == UNSUP
    assert create(lin(kind=1, scale=FAKE, xs=FAKE)) == UNSUP                      # W8A8
    assert create(lin(kind=2, K=128, scale=FAKE, group=128)) == UNSUP             # int4
    assert create(lin(splits=2, K=4096)) == UNSUP                                 # forced split
    assert create(lin(K=4104)) == UNSUP                                           # K > 4096
    assert create(lin(argmax_idx=FAKE)) == UNSUP                                  # epilogue
    # inputs against outputs: b reads 32 values (64 bytes) of a.y16 at various places
    y_b = FAKE + 0x20000
    for x_at, want in ((y16 + 64, "inside"), (y16 + 96, "straddles"), (y16 + 1, "odd")):
        b = lin(N=64, K=32, x=x_at, y=y_b)
        got = create(a, b)
        if want == "inside":
            assert got not in (UNSUP, SHAPE, NULL, ALIGN), got   # accepted by validation (fails later without a GPU)
        else:
            assert got in (UNSUP, ALIGN), (want, got)
    b = lin(N=64, K=32, x=y16, y=y_b)
    assert create(b, a) == UNSUP                                                  # reads a LATER linear's y16
    c = lin(N=64, K=64, x=y16, y=FAKE + 0x30000, y16_=y16)
    assert create(c) == UNSUP                                                     # reads its own y16
    d = lin(N=64, K=32, x=FAKE + 0x10000, y=y_b)
    assert create(a, d) == UNSUP                                                  # reads an fp32 y
    e = lin(N=64, K=64, x=FAKE + 0x40000, y=FAKE + 0x50000, y16_=y16 + 64)        # its y16 overlaps a's
    f = lin(N=64, K=64, x=y16 + 64, y=FAKE + 0x60000)                             # x inside both y16s
    assert create(a, e, f) == UNSUP
