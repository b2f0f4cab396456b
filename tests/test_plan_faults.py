"""Plan creation's failure paths and handle checks on the CPU.

With the test hooks enabled (WSG_ENABLE_TEST_HOOKS=1), wsg_decode_step_create
builds plans in host memory and can be made to fail at its device
allocation, its upload or its graph capture: every failure must return the
stated status, hand back no plan and free everything it made (the hooks count
the host blocks still alive).  A destroyed plan's handle is refused with
WSG_ERR_STATE by every call.  Pointers are fake device addresses that are
never dereferenced."""
import ctypes
import os

import pytest

from weight_streaming_gemv_decode_amd import wsgemv

FAKE = 0x7F0000000000
OK, NULL, SHAPE, ALIGN, UNSUP, WS, HIP, NOMEM, STATE = range(9)
NONE, ALLOC, UPLOAD, CAPTURE = 0, 1, 2, 3


@pytest.fixture()
def L():
    lib = wsgemv.lib()
    os.environ["WSG_ENABLE_TEST_HOOKS"] = "1"
    yield lib
    lib.wsg_test_set_fault(-1)
    os.environ.pop("WSG_ENABLE_TEST_HOOKS", None)


def _lins(n, kind=0, token=False):
    """n fp16 linears (or int4 / W8A8 ones), each with its own fake buffers."""
    out = []
    for i in range(n):
        base = FAKE + (i + 1) * 0x1000000
        if kind == 0:
            l = wsgemv.wsg_linear(0, 1, 300, 1024, base, None, base + 0x100000, None, base + 0x200000, None, 0, 0)
        elif kind == 1:
            l = wsgemv.wsg_linear(1, 1, 300, 2048, base, base + 0x300000, base + 0x100000, base + 0x400000,
                                  base + 0x200000, None, 0, 2)
        else:
            l = wsgemv.wsg_linear(2, 4, 300, 1024, base, base + 0x300000, base + 0x100000, None, base + 0x200000,
                                  None, 128, 0)
        if token and i == n - 1:
            l.argmax_idx = base + 0x500000
        out.append(l)
    return (wsgemv.wsg_linear * n)(*out)


def _chain(n):
    """n fp16 linears, each reading the previous one's y16 (persistent plans)."""
    out = []
    x = FAKE + 0x100000
    for i in range(n):
        base = FAKE + (i + 1) * 0x1000000
        l = wsgemv.wsg_linear(0, 1, 1024, 1024, base, None, x, None, base + 0x200000, None, 0, 0)
        l.y16 = base + 0x600000
        x = l.y16
        out.append(l)
    return (wsgemv.wsg_linear * n)(*out)


# every case needs a device block (token keys, split-K partials or work tables)
CASES = [("ordered graph", lambda: _lins(10, token=True), 0), ("ordered eager", lambda: _lins(3, token=True), 0x100),
         ("ordered forced graph", lambda: _lins(2, token=True), 0x200), ("grouped", lambda: _lins(5, token=True), 1),
         ("grouped mixed", lambda: _lins(3, kind=2), 1), ("ordered split w8a8", lambda: _lins(9, kind=1), 0),
         ("persistent", lambda: _chain(6), 2)]


def test_hooks_need_the_environment():
    lib = wsgemv.lib()
    os.environ.pop("WSG_ENABLE_TEST_HOOKS", None)
    assert lib.wsg_test_set_fault(0) == UNSUP


@pytest.mark.parametrize("name,make,mode", CASES, ids=[c[0] for c in CASES])
def test_host_plan_then_destroyed_handle(L, name, make, mode):
    assert L.wsg_test_set_fault(NONE) == OK
    arr = make()
    h = ctypes.c_void_p()
    assert L.wsg_decode_step_create(arr, len(arr), mode, None, ctypes.byref(h)) == OK
    assert h.value and L.wsg_test_live_blocks() == 1
    n, u, g = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int32()
    assert L.wsg_decode_step_info(h, ctypes.byref(n), ctypes.byref(u), ctypes.byref(g)) == OK
    assert n.value >= 1 and u.value >= 1 and g.value == 0
    assert L.decode_step_linears(h, None) == STATE        # a host-memory plan is never launched
    assert L.wsg_decode_step_destroy(h) == OK
    assert L.wsg_test_live_blocks() == 0
    # the destroyed handle is refused everywhere, not used
    assert L.decode_step_linears(h, None) == STATE
    assert L.wsg_decode_step_info(h, ctypes.byref(n), None, None) == STATE
    gu = ctypes.c_uint32()
    assert L.wsg_decode_step_status(h, None, ctypes.byref(gu)) == STATE
    assert L.wsg_decode_step_trace(h, None, 0) == STATE
    assert L.wsg_decode_step_destroy(h) == STATE
    assert L.wsg_decode_step_destroy(ctypes.c_void_p(FAKE)) == STATE   # never a plan


@pytest.mark.parametrize("name,make,mode", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("fault,want", [(ALLOC, NOMEM), (UPLOAD, HIP), (CAPTURE, HIP)])
def test_injected_failure_frees_everything(L, name, make, mode, fault, want):
    assert L.wsg_test_set_fault(fault) == OK
    arr = make()
    h = ctypes.c_void_p(12345)
    got = L.wsg_decode_step_create(arr, len(arr), mode, None, ctypes.byref(h))
    captures = (mode & 0xFF) != 2 and (mode & 0x100) == 0 and (mode == 0x200 or len(arr) >= 8 or name == "ordered split w8a8")
    if fault == CAPTURE and not captures:
        assert got == OK, got                               # no graph: nothing to capture
        assert L.wsg_decode_step_destroy(h) == OK
    else:
        assert got == want, (name, fault, got)
        assert not h.value                                  # no plan handed back
    assert L.wsg_test_live_blocks() == 0                    # and nothing left allocated


def test_trace_arguments(L):
    """wsg_decode_step_trace: persistent plans only; the buffer must be
    8-byte aligned and hold 4 words per work unit; NULL stops tracing."""
    assert L.wsg_test_set_fault(NONE) == OK
    h = ctypes.c_void_p()
    arr = _chain(4)
    assert L.wsg_decode_step_create(arr, len(arr), 2, None, ctypes.byref(h)) == OK
    u = ctypes.c_int64()
    assert L.wsg_decode_step_info(h, None, ctypes.byref(u), None) == OK
    n = 4 * u.value
    assert L.wsg_decode_step_trace(h, ctypes.c_void_p(FAKE + 4), n) == ALIGN
    assert L.wsg_decode_step_trace(h, ctypes.c_void_p(FAKE), n - 1) == SHAPE
    assert L.wsg_decode_step_trace(h, ctypes.c_void_p(FAKE), n) == OK
    assert L.wsg_decode_step_trace(h, None, 0) == OK
    assert L.wsg_decode_step_destroy(h) == OK
    g = ctypes.c_void_p()
    arr = _lins(3)
    assert L.wsg_decode_step_create(arr, len(arr), 1, None, ctypes.byref(g)) == OK
    assert L.wsg_decode_step_trace(g, ctypes.c_void_p(FAKE), 1 << 20) == UNSUP
    assert L.wsg_decode_step_destroy(g) == OK
    assert L.wsg_decode_step_trace(None, None, 0) == STATE
    assert L.wsg_test_live_blocks() == 0
