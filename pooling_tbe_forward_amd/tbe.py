"""Thin Python binding over libtbe.so, the C ABI declared in include/tbe.h.

Argument marshalling only: every step of the operator runs in the library's
HIP kernels.  PyTorch is used for device memory and streams.  The binding
fails loudly when the library has not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtbe.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "tbe.h")

TBE_OK, TBE_EINVAL, TBE_ERANGE, TBE_ENOMEM, TBE_EHIP, TBE_ENOTSUP = range(6)
TBE_F32, TBE_F16 = 0, 1
TBE_I32, TBE_I64 = 0, 1

_lib = None


class TBEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {tbe_status_string(status)} (status {status})")


class tbe_tuning(ctypes.Structure):
    _fields_ = [("tau", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("hist_mode", ctypes.c_int32), ("hist_min_mean_len", ctypes.c_int32),
                ("fwd_bags_per_wave", ctypes.c_int32), ("seg_slab_kib", ctypes.c_int32),
                ("sort_mode", ctypes.c_int32), ("reserved", ctypes.c_int32 * 9)]


class tbe_sort_view(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("sorted_keys", "sorted_pos", "unique_keys", "run_start", "run_len",
                 "short_runs", "long_runs", "counts")]


def lib():
    """Load libtbe.so (raises if it is missing: build it first)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m pooling_tbe_forward_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.tbe_plan_create.argtypes = [I32, P, P, I32, I32, P, ctypes.POINTER(P)]
        L.tbe_plan_create.restype = I32
        L.tbe_plan_destroy.argtypes = [P]
        L.tbe_plan_destroy.restype = None
        L.tbe_plan_layout.argtypes = [P, P, P, P]
        L.tbe_plan_layout.restype = I32
        L.tbe_forward.argtypes = [P, I32, P, P, I64, P, P, P, P]
        L.tbe_forward.restype = I32
        L.tbe_backward_workspace_bytes.argtypes = [P, I32, I64]
        L.tbe_backward_workspace_bytes.restype = SZ
        L.tbe_backward_sgd.argtypes = [P, I32, P, P, I64, P, P, P, ctypes.c_float, P, SZ, P]
        L.tbe_backward_sgd.restype = I32
        L.tbe_backward_sgd_noalloc.argtypes = [P, I32, P, P, I64, P, P, P, ctypes.c_float, P, P]
        L.tbe_backward_sgd_noalloc.restype = I32
        L.tbe_backward_noalloc_max_bytes.argtypes = []
        L.tbe_backward_noalloc_max_bytes.restype = SZ
        L.tbe_backward_prepare.argtypes = [P, I32, P, I64, P, P, P, SZ, P]
        L.tbe_backward_prepare.restype = I32
        L.tbe_backward_apply.argtypes = [P, I32, I64, I32, P, P, ctypes.c_float, P, SZ, P]
        L.tbe_backward_apply.restype = I32
        F = ctypes.c_float
        L.tbe_backward_adagrad.argtypes = [P, I32, P, P, P, I64, P, P, P, F, F, P, SZ, P]
        L.tbe_backward_adagrad.restype = I32
        L.tbe_backward_apply_adagrad.argtypes = [P, I32, I64, I32, P, P, P, F, F, P, SZ, P]
        L.tbe_backward_apply_adagrad.restype = I32
        L.tbe_sort_rle.argtypes = [P, I32, P, I64, P, P, SZ, ctypes.POINTER(tbe_sort_view), P]
        L.tbe_sort_rle.restype = I32
        L.tbe_set_stage_events.argtypes = [P, ctypes.POINTER(ctypes.c_void_p), I32]
        L.tbe_set_stage_events.restype = I32
        L.tbe_workspace_init.argtypes = [P, SZ, P]
        L.tbe_workspace_init.restype = I32
        L.tbe_workspace_status.argtypes = [P, SZ, P, P]
        L.tbe_workspace_status.restype = I32
        L.tbe_bounds_check.argtypes = [P, I32, P, I64, P, P, P]
        L.tbe_bounds_check.restype = I32
        L.tbe_get_tuning.argtypes = [P, ctypes.POINTER(tbe_tuning)]
        L.tbe_get_tuning.restype = I32
        L.tbe_set_tuning.argtypes = [P, ctypes.POINTER(tbe_tuning)]
        L.tbe_set_tuning.restype = I32
        L.tbe_plan_set_pooling.argtypes = [P, I32]
        L.tbe_plan_set_pooling.restype = I32
        L.tbe_status_string.argtypes = [I32]
        L.tbe_status_string.restype = ctypes.c_char_p
        L.tbe_version.argtypes = []
        L.tbe_version.restype = I32
        _lib = L
    return _lib


def header_symbols():
    """Function names declared in include/tbe.h."""
    src = open(HEADER_PATH).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tbe_[a-z_]+)\s*\(", src)))


def tbe_status_string(status: int) -> str:
    return lib().tbe_status_string(int(status)).decode()


def tbe_version() -> int:
    return int(lib().tbe_version())


def _check(status: int, where: str):
    if status != TBE_OK:
        raise TBEError(status, where)


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype, numel=None, at_least=False):
    """Raise unless tensor t has this dtype and size: the kernels read every
    buffer at the widths and lengths the plan implies."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and (t.numel() < numel if at_least else t.numel() != numel):
        raise ValueError(f"{name} must have {'at least ' if at_least else ''}{numel} "
                         f"elements, got {t.numel()}")


def _check_jagged(plan, B, indices, offsets, per_sample_weights=None):
    it = plan.torch_idtype
    _need(indices, "indices", it)
    _need(offsets, "offsets", it, plan.T * int(B) + 1)
    if per_sample_weights is not None:
        _need(per_sample_weights, "per_sample_weights", torch.float32, indices.numel())


def _check_dense(plan, B, weights=None, rowmajor=None, rowmajor_name="grad_output"):
    if weights is not None or rowmajor is None:
        _need(weights, "weights", plan.torch_wdtype, plan.weight_elems, at_least=True)
    if rowmajor is not None:
        _need(rowmajor, rowmajor_name, torch.float32, int(B) * plan.sum_D)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Plan:
    """Owns a tbe_plan*; destroyed with the object."""

    def __init__(self, handle, T, rows, dims, weight_dtype, index_dtype):
        self.handle = handle
        self.T = T
        self.rows = list(rows)
        self.dims = list(dims)
        self.weight_dtype = weight_dtype
        self.index_dtype = index_dtype
        self.sum_D = sum(self.dims)
        self.sum_rows = sum(self.rows)
        self.weight_elems = sum(r * d for r, d in zip(self.rows, self.dims))

    @property
    def torch_wdtype(self):
        return torch.float32 if self.weight_dtype == TBE_F32 else torch.float16

    @property
    def torch_idtype(self):
        return torch.int32 if self.index_dtype == TBE_I32 else torch.int64

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        if h and _lib is not None:
            _lib.tbe_plan_destroy(h)


def tbe_plan_create(rows, dims, weight_dtype=TBE_F32, index_dtype=TBE_I32, weighted=None) -> Plan:
    rows = [int(r) for r in rows]
    dims = [int(d) for d in dims]
    T = len(rows)
    r = (ctypes.c_int64 * T)(*rows)
    d = (ctypes.c_int32 * len(dims))(*dims)
    w = None if weighted is None else (ctypes.c_uint8 * T)(*[1 if x else 0 for x in weighted])
    h = ctypes.c_void_p()
    _check(lib().tbe_plan_create(T, r, d, int(weight_dtype), int(index_dtype), w, ctypes.byref(h)),
           "tbe_plan_create")
    return Plan(h, T, rows, dims, weight_dtype, index_dtype)


def tbe_plan_layout(plan: Plan):
    T = plan.T
    wo = (ctypes.c_int64 * T)()
    do = (ctypes.c_int64 * (T + 1))()
    hc = (ctypes.c_int64 * (T + 1))()
    _check(lib().tbe_plan_layout(plan.handle, wo, do, hc), "tbe_plan_layout")
    return list(wo), list(do), list(hc)


def tbe_get_tuning(plan: Plan) -> tbe_tuning:
    t = tbe_tuning()
    _check(lib().tbe_get_tuning(plan.handle, ctypes.byref(t)), "tbe_get_tuning")
    return t


POOLING = {"sum": 0, "mean": 1}


def tbe_plan_set_pooling(plan: Plan, pooling: str):
    """"sum" (default) or "mean": a bag's sum divided by its length."""
    _check(lib().tbe_plan_set_pooling(plan.handle, POOLING[pooling]), "tbe_plan_set_pooling")


def tbe_set_tuning(plan: Plan, **kw):
    t = tbe_get_tuning(plan)
    for k, v in kw.items():
        setattr(t, k, int(v))
    _check(lib().tbe_set_tuning(plan.handle, ctypes.byref(t)), "tbe_set_tuning")
    return t


def tbe_forward(plan: Plan, B: int, weights, indices, offsets, per_sample_weights, output,
                stream=None):
    _check_jagged(plan, B, indices, offsets, per_sample_weights)
    _check_dense(plan, B, weights, output, "output")
    _check(lib().tbe_forward(plan.handle, int(B), _ptr(weights), _ptr(indices),
                             int(indices.numel()), _ptr(offsets), _ptr(per_sample_weights),
                             _ptr(output), _stream(stream)), "tbe_forward")
    return output


def tbe_backward_workspace_bytes(plan: Plan, B: int, num_indices: int) -> int:
    return int(lib().tbe_backward_workspace_bytes(plan.handle, int(B), int(num_indices)))


def tbe_set_stage_events(plan: Plan, events):
    """events: sequence of raw hipEvent_t handles (ints, None for a stage not
    recorded); an empty sequence or None clears."""
    if not events:
        _check(lib().tbe_set_stage_events(plan.handle, None, 0), "tbe_set_stage_events")
        return
    arr = (ctypes.c_void_p * len(events))(*events)
    _check(lib().tbe_set_stage_events(plan.handle, arr, len(events)), "tbe_set_stage_events")


def tbe_workspace_init(workspace, stream=None):
    _check(lib().tbe_workspace_init(_ptr(workspace),
                                    int(workspace.numel() * workspace.element_size()),
                                    _stream(stream)), "tbe_workspace_init")
    return workspace


def alloc_workspace(plan: Plan, B: int, num_indices: int, device="cuda"):
    """Allocate (through torch) and initialise a backward workspace."""
    n = tbe_backward_workspace_bytes(plan, B, num_indices)
    if n == 0:
        raise TBEError(TBE_EINVAL, "tbe_backward_workspace_bytes")
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    return tbe_workspace_init(ws)


def tbe_backward_sgd(plan: Plan, B: int, weights, indices, offsets, per_sample_weights,
                     grad_output, lr: float, workspace, stream=None):
    _check_jagged(plan, B, indices, offsets, per_sample_weights)
    _check_dense(plan, B, weights, grad_output)
    _check(lib().tbe_backward_sgd(plan.handle, int(B), _ptr(weights), _ptr(indices),
                                  int(indices.numel()), _ptr(offsets), _ptr(per_sample_weights),
                                  _ptr(grad_output), float(lr), _ptr(workspace),
                                  int(workspace.numel() * workspace.element_size()),
                                  _stream(stream)), "tbe_backward_sgd")
    return weights


def tbe_backward_sgd_noalloc(plan: Plan, B: int, weights, indices, offsets, per_sample_weights,
                             grad_output, lr: float, error_word=None, stream=None):
    """tbe_backward_sgd with the library's own per-GPU workspace array (no
    allocation by the library or the binding).  error_word: optional device
    int32 tensor of one element that receives the call's error word."""
    _check_jagged(plan, B, indices, offsets, per_sample_weights)
    _check_dense(plan, B, weights, grad_output)
    if error_word is not None:
        _need(error_word, "error_word", torch.int32, 1)
    _check(lib().tbe_backward_sgd_noalloc(plan.handle, int(B), _ptr(weights), _ptr(indices),
                                          int(indices.numel()), _ptr(offsets),
                                          _ptr(per_sample_weights), _ptr(grad_output), float(lr),
                                          _ptr(error_word), _stream(stream)),
           "tbe_backward_sgd_noalloc")
    return weights


def tbe_backward_noalloc_max_bytes() -> int:
    return int(lib().tbe_backward_noalloc_max_bytes())


def tbe_backward_prepare(plan: Plan, B: int, indices, offsets, per_sample_weights, workspace,
                         stream=None):
    _check_jagged(plan, B, indices, offsets, per_sample_weights)
    _check(lib().tbe_backward_prepare(plan.handle, int(B), _ptr(indices), int(indices.numel()),
                                      _ptr(offsets), _ptr(per_sample_weights), _ptr(workspace),
                                      int(workspace.numel() * workspace.element_size()),
                                      _stream(stream)), "tbe_backward_prepare")
    return workspace


def tbe_backward_apply(plan: Plan, B: int, num_indices: int, weighted: bool, weights,
                       grad_output, lr: float, workspace, stream=None):
    _check_dense(plan, B, weights, grad_output)
    _check(lib().tbe_backward_apply(plan.handle, int(B), int(num_indices), 1 if weighted else 0,
                                    _ptr(weights), _ptr(grad_output), float(lr), _ptr(workspace),
                                    int(workspace.numel() * workspace.element_size()),
                                    _stream(stream)), "tbe_backward_apply")
    return weights


ADAGRAD_EPS = 1e-8   # the pages give no value for eps


def tbe_backward_adagrad(plan: Plan, B: int, weights, state, indices, offsets,
                         per_sample_weights, grad_output, lr: float, workspace,
                         eps: float = ADAGRAD_EPS, stream=None):
    """Backward + exact row-wise Adagrad in place; ``state`` is the fp32 row
    state, one value per row of every table (indexed by the row's key)."""
    _check_jagged(plan, B, indices, offsets, per_sample_weights)
    _check_dense(plan, B, weights, grad_output)
    _need(state, "state", torch.float32, plan.sum_rows)
    _check(lib().tbe_backward_adagrad(plan.handle, int(B), _ptr(weights), _ptr(state),
                                      _ptr(indices), int(indices.numel()), _ptr(offsets),
                                      _ptr(per_sample_weights), _ptr(grad_output), float(lr),
                                      float(eps), _ptr(workspace),
                                      int(workspace.numel() * workspace.element_size()),
                                      _stream(stream)), "tbe_backward_adagrad")
    return weights


def tbe_backward_apply_adagrad(plan: Plan, B: int, num_indices: int, weighted: bool, weights,
                               state, grad_output, lr: float, workspace,
                               eps: float = ADAGRAD_EPS, stream=None):
    _check_dense(plan, B, weights, grad_output)
    _need(state, "state", torch.float32, plan.sum_rows)
    _check(lib().tbe_backward_apply_adagrad(plan.handle, int(B), int(num_indices),
                                            1 if weighted else 0, _ptr(weights), _ptr(state),
                                            _ptr(grad_output), float(lr), float(eps),
                                            _ptr(workspace),
                                            int(workspace.numel() * workspace.element_size()),
                                            _stream(stream)), "tbe_backward_apply_adagrad")
    return weights


def tbe_sort_rle(plan: Plan, B: int, indices, offsets, workspace, stream=None) -> dict:
    """Returns int32 tensors viewing the workspace (keys as unsigned 32-bit
    values stored in int32) plus the device counts tensor."""
    _check_jagged(plan, B, indices, offsets)
    v = tbe_sort_view()
    N = int(indices.numel())
    _check(lib().tbe_sort_rle(plan.handle, int(B), _ptr(indices), N, _ptr(offsets),
                              _ptr(workspace), int(workspace.numel() * workspace.element_size()),
                              ctypes.byref(v), _stream(stream)), "tbe_sort_rle")
    base = workspace.data_ptr()
    raw = workspace.view(torch.uint8)

    def view(ptr, n):
        off = int(ptr) - base
        return raw[off:off + 4 * n].view(torch.int32)

    return dict(sorted_keys=view(v.sorted_keys, N), sorted_pos=view(v.sorted_pos, N),
                unique_keys=view(v.unique_keys, N), run_start=view(v.run_start, N + 1),
                run_len=view(v.run_len, N), short_runs=view(v.short_runs, N),
                long_runs=view(v.long_runs, N), counts=view(v.counts, 6))


def tbe_workspace_status(workspace, error_word=None, stream=None):
    """Enqueue a copy of the workspace's error word (TBE_WS_ERR_* bits) into
    ``error_word`` (a device int32 tensor of one element; allocated when not
    given) and return that tensor; read it after the stream is synchronised."""
    if error_word is None:
        error_word = torch.zeros(1, dtype=torch.int32, device=workspace.device)
    _need(error_word, "error_word", torch.int32, 1)
    _check(lib().tbe_workspace_status(_ptr(workspace),
                                      int(workspace.numel() * workspace.element_size()),
                                      _ptr(error_word), _stream(stream)), "tbe_workspace_status")
    return error_word


TBE_WS_ERR_LOOKBACK, TBE_WS_ERR_CONTROL, TBE_WS_ERR_PAYLOAD = 1, 2, 4


def tbe_bounds_check(plan: Plan, B: int, indices, offsets, error_count, stream=None):
    _need(indices, "indices", plan.torch_idtype)
    _need(offsets, "offsets", plan.torch_idtype, plan.T * int(B) + 1)
    _need(error_count, "error_count", torch.int64, 1, at_least=True)
    _check(lib().tbe_bounds_check(plan.handle, int(B), _ptr(indices), int(indices.numel()),
                                  _ptr(offsets), _ptr(error_count), _stream(stream)),
           "tbe_bounds_check")
    return error_count
