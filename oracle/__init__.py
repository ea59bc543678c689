"""CPU oracle for the table-batched embedding-bag (TBE) operator.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may use it; the product path never does.  It
shares no code with the HIP library: the arithmetic lives in ``oracle.c``
(plain C, double accumulation) and this module only marshals numpy arrays.

What each function computes, and the passage of the FBTriton TBE article it
follows, is documented in ``oracle.h``.  Every function here is pinned by the
CPU tests (hand-worked example, dense one-hot brute force, library special
cases, exact-arithmetic invariants); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_HDR = os.path.join(_HERE, "oracle.h")
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, F16 = 0, 1
POOLING = {"sum": 0, "mean": 1}


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (fast); skipped when it is up to date."""
    if (not force and os.path.exists(_SO)
            and os.path.getmtime(_SO) >= max(os.path.getmtime(_SRC), os.path.getmtime(_HDR))):
        return _SO
    tmp = _SO + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-Wall", "-fPIC", "-shared", "-fopenmp",
                           _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _SO)
    return _SO


class _Table(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("ids", ctypes.c_void_p), ("data", ctypes.c_void_p)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        L.oracle_layout.argtypes = [ctypes.c_int32, P, P, P, P, P]
        L.oracle_forward.argtypes = [ctypes.c_int32, ctypes.c_int32, P, P, ctypes.c_int32,
                                     P, P, P, P, P, P, ctypes.c_int64, P, ctypes.c_int32]
        L.oracle_sort_rle.argtypes = [ctypes.c_int32, ctypes.c_int32, P, P, P, ctypes.c_int64,
                                      P, P, P, P, P, P, P, P, P, P]
        L.oracle_backward_sgd.argtypes = [ctypes.c_int32, ctypes.c_int32, P, P, ctypes.c_int32,
                                          P, P, P, P, P, P, ctypes.c_float, P, ctypes.c_int64,
                                          P, P, ctypes.c_int32, ctypes.c_int32]
        L.oracle_backward_adagrad.argtypes = [ctypes.c_int32, ctypes.c_int32, P, P,
                                              ctypes.c_int32, P, P, P, P, P, P, ctypes.c_float,
                                              ctypes.c_float, P, ctypes.c_int64, P, P, P, P,
                                              ctypes.c_int32, ctypes.c_int32]
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        L.oracle_set_threads.restype = ctypes.c_int
        L.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_half_to_double.restype = ctypes.c_double
        L.oracle_double_to_half.argtypes = [ctypes.c_double]
        L.oracle_double_to_half.restype = ctypes.c_uint16
        _lib = L
    return _lib


class OracleError(RuntimeError):
    pass


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc):
    if rc != 0:
        raise OracleError({1: "invalid argument", 2: "input out of range",
                           3: "row not held"}.get(rc, str(rc)))


def _i64(a):
    return np.ascontiguousarray(a, dtype=np.int64)


def _tables(tables, dims, wdtype):
    """tables: list of (ids or None, data array [n, D] or flat)."""
    npdt = np.float32 if wdtype == F32 else np.float16
    arr = (_Table * len(tables))()
    keep = []
    for t, (ids, data) in enumerate(tables):
        assert data.dtype == npdt and data.flags.c_contiguous
        n = data.size // int(dims[t])
        arr[t].n = n
        if ids is not None:
            ids = _i64(ids)
            assert ids.size == n
            keep.append(ids)
            arr[t].ids = ids.ctypes.data
        else:
            arr[t].ids = None
        arr[t].data = data.ctypes.data
    return arr, keep


def layout(rows, dims):
    rows = _i64(rows)
    dims = np.ascontiguousarray(dims, dtype=np.int32)
    T = rows.size
    wo = np.zeros(T, np.int64)
    do = np.zeros(T + 1, np.int64)
    hc = np.zeros(T + 1, np.int64)
    _check(lib().oracle_layout(T, _p(rows), _p(dims), _p(wo), _p(do), _p(hc)))
    return wo, do, hc


def dense_tables(packed, rows, dims):
    """Split a packed host weight array into per-table dense views."""
    wo, _, _ = layout(rows, dims)
    out = []
    for t in range(len(rows)):
        n = int(rows[t]) * int(dims[t])
        out.append((None, packed[int(wo[t]):int(wo[t]) + n]))
    return out


def forward(T, B, rows, dims, wdtype, tables, indices, offsets, psw=None,
            weighted=None, bag_list=None, pooling="sum"):
    """Pooled forward in float64 (pooling "sum" or "mean").  Returns
    [B, sum D], or [len(bag_list), Dmax]."""
    rows = _i64(rows)
    dims = np.ascontiguousarray(dims, dtype=np.int32)
    indices = _i64(indices)
    offsets = _i64(offsets)
    psw = None if psw is None else np.ascontiguousarray(psw, dtype=np.float32)
    wm = None if weighted is None else np.ascontiguousarray(weighted, dtype=np.uint8)
    tarr, keep = _tables(tables, dims, wdtype)
    if bag_list is None:
        out = np.zeros((B, int(dims.sum())), np.float64)
        bl, nb = None, 0
    else:
        bl = _i64(bag_list)
        nb = bl.size
        out = np.zeros((nb, int(dims.max())), np.float64)
    _check(lib().oracle_forward(T, B, _p(rows), _p(dims), wdtype, ctypes.cast(tarr, ctypes.c_void_p),
                                _p(indices), _p(offsets), _p(psw), _p(wm), _p(bl), nb, _p(out),
                                POOLING[pooling]))
    del keep
    return out


def sort_rle(T, B, rows, indices, offsets, tau):
    rows = _i64(rows)
    indices = _i64(indices)
    offsets = _i64(offsets)
    N = int(offsets[-1])
    n1 = max(N, 1)
    r = {k: np.zeros(n1, np.int64) for k in
         ("sorted_keys", "sorted_pos", "unique_keys", "run_start", "run_len",
          "short_runs", "long_runs")}
    cnt = {k: np.zeros(1, np.int64) for k in ("num_runs", "num_short", "num_long")}
    _check(lib().oracle_sort_rle(T, B, _p(rows), _p(indices), _p(offsets), int(tau),
                                 _p(r["sorted_keys"]), _p(r["sorted_pos"]), _p(r["unique_keys"]),
                                 _p(r["run_start"]), _p(r["run_len"]), _p(cnt["num_runs"]),
                                 _p(r["short_runs"]), _p(cnt["num_short"]),
                                 _p(r["long_runs"]), _p(cnt["num_long"])))
    R, S, Lg = int(cnt["num_runs"][0]), int(cnt["num_short"][0]), int(cnt["num_long"][0])
    return dict(sorted_keys=r["sorted_keys"][:N], sorted_pos=r["sorted_pos"][:N],
                unique_keys=r["unique_keys"][:R], run_start=r["run_start"][:R],
                run_len=r["run_len"][:R], num_runs=R,
                short_runs=r["short_runs"][:S], long_runs=r["long_runs"][:Lg],
                num_short=S, num_long=Lg)


def backward_sgd(T, B, rows, dims, wdtype, tables, indices, offsets, psw, weighted,
                 grad_output, lr, keys, write_back=False, pooling="sum"):
    """Finished row gradients and exact SGD rows (float64) for ``keys``.

    Returns (grad_rows [nkeys, Dmax], new_rows [nkeys, Dmax]).  With
    write_back, the rounded rows are stored into the tables' host arrays."""
    rows = _i64(rows)
    dims = np.ascontiguousarray(dims, dtype=np.int32)
    indices = _i64(indices)
    offsets = _i64(offsets)
    psw = None if psw is None else np.ascontiguousarray(psw, dtype=np.float32)
    wm = None if weighted is None else np.ascontiguousarray(weighted, dtype=np.uint8)
    g = np.ascontiguousarray(grad_output, dtype=np.float32)
    keys = _i64(keys)
    tarr, keep = _tables(tables, dims, wdtype)
    Dmax = int(dims.max())
    gr = np.zeros((keys.size, Dmax), np.float64)
    nr = np.zeros((keys.size, Dmax), np.float64)
    _check(lib().oracle_backward_sgd(T, B, _p(rows), _p(dims), wdtype,
                                     ctypes.cast(tarr, ctypes.c_void_p), _p(indices), _p(offsets),
                                     _p(psw), _p(wm), _p(g), float(lr), _p(keys), keys.size,
                                     _p(gr), _p(nr), 1 if write_back else 0, POOLING[pooling]))
    del keep
    return gr, nr


def backward_adagrad(T, B, rows, dims, wdtype, tables, indices, offsets, psw, weighted,
                      grad_output, lr, eps, keys, state_in, write_back=False, pooling="sum"):
    """Finished row gradients, exact row-wise Adagrad rows (float64) and the
    rows' new fp32 state for ``keys``; ``state_in`` is the state of each
    key's row before the step.

    Returns (grad_rows [nkeys, Dmax], new_rows [nkeys, Dmax], state_out
    [nkeys] float32).  With write_back, the rounded rows are stored into the
    tables' host arrays."""
    rows = _i64(rows)
    dims = np.ascontiguousarray(dims, dtype=np.int32)
    indices = _i64(indices)
    offsets = _i64(offsets)
    psw = None if psw is None else np.ascontiguousarray(psw, dtype=np.float32)
    wm = None if weighted is None else np.ascontiguousarray(weighted, dtype=np.uint8)
    g = np.ascontiguousarray(grad_output, dtype=np.float32)
    keys = _i64(keys)
    s_in = np.ascontiguousarray(state_in, dtype=np.float32)
    if s_in.shape != keys.shape:
        raise ValueError("state_in needs one value per key")
    tarr, keep = _tables(tables, dims, wdtype)
    Dmax = int(dims.max())
    gr = np.zeros((keys.size, Dmax), np.float64)
    nr = np.zeros((keys.size, Dmax), np.float64)
    s_out = np.zeros(keys.size, np.float32)
    _check(lib().oracle_backward_adagrad(T, B, _p(rows), _p(dims), wdtype,
                                         ctypes.cast(tarr, ctypes.c_void_p), _p(indices),
                                         _p(offsets), _p(psw), _p(wm), _p(g), float(lr),
                                         float(eps), _p(keys), keys.size, _p(s_in), _p(s_out),
                                         _p(gr), _p(nr), 1 if write_back else 0,
                                         POOLING[pooling]))
    del keep
    return gr, nr, s_out


def set_threads(n: int) -> int:
    """Host threads for forward and backward (1 = single-threaded, the
    default); results are the same bits for any count."""
    return int(lib().oracle_set_threads(int(n)))


def half_to_double(bits):
    L = lib()
    return np.array([L.oracle_half_to_double(int(b)) for b in np.asarray(bits).ravel()],
                    dtype=np.float64)


def double_to_half(vals):
    L = lib()
    return np.array([L.oracle_double_to_half(float(v)) for v in np.asarray(vals).ravel()],
                    dtype=np.uint16)
