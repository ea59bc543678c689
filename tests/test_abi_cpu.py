"""C-ABI library checks that need no GPU: it loads, exports every function
include/tbe.h declares, and rejects host-checkable bad arguments before
touching the device."""
import ctypes

import pytest

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
    assert tbe.tbe_version() == 100


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
