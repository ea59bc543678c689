"""C-ABI library checks that need no GPU: it loads, exports every function
include/tbe.h declares, and rejects host-checkable bad arguments before
touching the device."""
import ctypes

import pytest
import torch

from pooling_tbe_forward_amd import tbe


def test_exports_every_declared_symbol():
    L = tbe.lib()
    names = tbe.header_symbols()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version():
    seen = set()
    for s in range(6):
        txt = tbe.tbe_status_string(s)
        assert txt and txt not in seen
        seen.add(txt)
    assert tbe.tbe_status_string(99) == "unknown status"
    assert tbe.tbe_version() == 101


def _create(T, rows, dims, wd=0, it=0, out=True):
    L = tbe.lib()
    r = (ctypes.c_int64 * max(T, 1))(*rows)
    d = (ctypes.c_int32 * max(T, 1))(*dims)
    h = ctypes.c_void_p()
    return L.tbe_plan_create(T, r, d, wd, it, None, ctypes.byref(h) if out else None)


def test_plan_create_rejects_bad_arguments():
    assert _create(0, [1], [1]) == tbe.TBE_EINVAL            # no tables
    assert _create(1, [1], [1], out=False) == tbe.TBE_EINVAL  # no output slot
    assert _create(1, [1], [0]) == tbe.TBE_EINVAL            # D = 0
    assert _create(1, [-1], [4]) == tbe.TBE_EINVAL           # negative rows
    assert _create(1, [1], [4], wd=7) == tbe.TBE_EINVAL      # bad weight dtype
    assert _create(1, [1], [4], it=3) == tbe.TBE_EINVAL      # bad index dtype
    assert _create(1, [1], [5000]) == tbe.TBE_ERANGE         # D above 4096
    assert _create(2, [1 << 31, 1 << 31], [4, 4]) == tbe.TBE_ERANGE  # keys need > 32 bits


def test_null_plan_calls():
    L = tbe.lib()
    assert L.tbe_forward(None, 1, None, None, 0, None, None, None, None) == tbe.TBE_EINVAL
    assert L.tbe_backward_workspace_bytes(None, 1, 10) == 0
    assert L.tbe_backward_sgd(None, 1, None, None, 0, None, None, None, 0.1, None, 0,
                              None) == tbe.TBE_EINVAL
    assert L.tbe_bounds_check(None, 1, None, 0, None, None, None) == tbe.TBE_EINVAL
    assert L.tbe_set_tuning(None, None) == tbe.TBE_EINVAL
    assert L.tbe_plan_set_pooling(None, 1) == tbe.TBE_EINVAL
    assert L.tbe_plan_layout(None, None, None, None) == tbe.TBE_EINVAL
    assert L.tbe_workspace_init(None, 1 << 20, None) == tbe.TBE_EINVAL
    assert L.tbe_set_stage_events(None, None, 0) == tbe.TBE_EINVAL
    assert L.tbe_backward_prepare(None, 1, None, 0, None, None, None, 0, None) == tbe.TBE_EINVAL
    assert L.tbe_backward_apply(None, 1, 0, 0, None, None, 0.1, None, 0, None) == tbe.TBE_EINVAL
    assert L.tbe_backward_adagrad(None, 1, None, None, None, 0, None, None, None, 0.1, 1e-8,
                                  None, 0, None) == tbe.TBE_EINVAL
    assert L.tbe_backward_apply_adagrad(None, 1, 0, 0, None, None, None, 0.1, 1e-8, None, 0,
                                        None) == tbe.TBE_EINVAL
    L.tbe_plan_destroy(None)


def test_binding_raises():
    with pytest.raises(tbe.TBEError) as e:
        tbe.tbe_plan_create([], [])
    assert e.value.status == tbe.TBE_EINVAL


def test_workspace_status_rejects_bad_arguments():
    """Host-checkable arguments of the error-word accessor are refused before
    anything is enqueued (none of these pointers is dereferenced)."""
    L = tbe.lib()
    ws = ctypes.c_void_p(1 << 20)          # 256-byte aligned stand-in, never read
    word = ctypes.c_void_p(1 << 12)
    big = 1 << 20
    assert L.tbe_workspace_status(None, big, word, None) == tbe.TBE_EINVAL
    assert L.tbe_workspace_status(ctypes.c_void_p((1 << 20) + 4), big, word,
                                  None) == tbe.TBE_EINVAL     # misaligned workspace
    assert L.tbe_workspace_status(ws, 1024, word, None) == tbe.TBE_EINVAL   # smaller than control block
    assert L.tbe_workspace_status(ws, big, None, None) == tbe.TBE_EINVAL
    assert L.tbe_workspace_status(ws, big, ctypes.c_void_p((1 << 12) + 2),
                                  None) == tbe.TBE_EINVAL     # misaligned word


def _host_plan(wd=tbe.TBE_F32, it=tbe.TBE_I32):
    # a Plan object with no library handle: the binding's checks run first
    return tbe.Plan(None, 2, [10, 5], [4, 8], wd, it)


def test_binding_checks_dtypes_and_sizes():
    """The binding refuses tensors whose dtype or length does not match the
    plan, before any call reaches the library (the kernels would read them at
    the plan's widths)."""
    p = _host_plan()
    B = 3
    ok = dict(weights=torch.zeros(10 * 4 + 5 * 8), indices=torch.zeros(7, dtype=torch.int32),
              offsets=torch.zeros(2 * B + 1, dtype=torch.int32), psw=torch.zeros(7),
              out=torch.zeros(B, 12), grad=torch.zeros(B, 12))

    def fwd(**kw):
        a = {**ok, **kw}
        tbe.tbe_forward(p, B, a["weights"], a["indices"], a["offsets"], a["psw"], a["out"])

    def bwd(**kw):
        a = {**ok, **kw}
        tbe.tbe_backward_sgd(p, B, a["weights"], a["indices"], a["offsets"], a["psw"], a["grad"],
                             0.1, torch.zeros(64, dtype=torch.uint8))

    for call in (fwd, bwd):
        with pytest.raises(TypeError):
            call(indices=torch.zeros(7, dtype=torch.int64))        # plan says int32
        with pytest.raises(TypeError):
            call(offsets=torch.zeros(2 * B + 1, dtype=torch.int64))
        with pytest.raises(ValueError):
            call(offsets=torch.zeros(2 * B, dtype=torch.int32))    # T*B+1 entries needed
        with pytest.raises(TypeError):
            call(weights=torch.zeros(80, dtype=torch.float16))     # plan says fp32
        with pytest.raises(ValueError):
            call(weights=torch.zeros(79))                          # fewer than sum rows*D
        with pytest.raises(ValueError):
            call(psw=torch.zeros(6))                               # one per lookup
        with pytest.raises(TypeError):
            call(psw=torch.zeros(7, dtype=torch.float64))
    with pytest.raises(ValueError):
        fwd(out=torch.zeros(B, 11))                                # [B, sum D]
    with pytest.raises(ValueError):
        bwd(grad=torch.zeros(B + 1, 12))
    with pytest.raises(ValueError, match="GPU"):
        fwd()                                                      # shapes fine: CPU tensors refused
    with pytest.raises(ValueError):
        tbe.tbe_backward_adagrad(p, B, ok["weights"], torch.zeros(14), ok["indices"],
                                 ok["offsets"], None, ok["grad"], 0.1,
                                 torch.zeros(64, dtype=torch.uint8))   # one state per row: 15
    with pytest.raises(TypeError):
        tbe.tbe_bounds_check(p, B, ok["indices"], ok["offsets"],
                             torch.zeros(1, dtype=torch.int32))
