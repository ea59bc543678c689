"""Glue between the seeded problems and the CPU oracle / the HIP binding.

Only marshalling lives here: the arithmetic under test is in ``oracle/`` (CPU)
and in the HIP library (GPU).
"""
from __future__ import annotations

import numpy as np

import oracle
from pooling_tbe_forward_amd import datagen as dg


def wcode(prob):
    return oracle.F32 if prob.wdtype == "f32" else oracle.F16


def oracle_forward(prob, packed, bag_list=None):
    tabs = oracle.dense_tables(packed, prob.rows, prob.dims)
    return oracle.forward(prob.T, prob.B, prob.rows, prob.dims, wcode(prob), tabs,
                          prob.indices, prob.offsets, prob.psw, prob.weighted,
                          bag_list=bag_list)


def oracle_sort(prob, tau):
    return oracle.sort_rle(prob.T, prob.B, prob.rows, prob.indices, prob.offsets, tau)


def oracle_backward(prob, packed, keys=None, write_back=True, lr=None):
    """Run the backward-SGD oracle on a packed host weight copy (modified in
    place when write_back).  Returns (keys, grad_rows, new_rows)."""
    if keys is None:
        keys = oracle_sort(prob, 1 << 62)["unique_keys"]
    tabs = oracle.dense_tables(packed, prob.rows, prob.dims)
    gr, nr = oracle.backward_sgd(prob.T, prob.B, prob.rows, prob.dims, wcode(prob), tabs,
                                 prob.indices, prob.offsets, prob.psw, prob.weighted,
                                 prob.grad, prob.lr if lr is None else lr, keys,
                                 write_back=write_back)
    return keys, gr, nr


def sparse_tables(prob, row_sets):
    """Per-table sparse row stores generated on the host: row_sets[t] is a
    sorted unique int64 array of row ids."""
    out = []
    for t in range(prob.T):
        ids = np.asarray(row_sets[t], dtype=np.int64)
        data = np.ascontiguousarray(dg.weight_rows(prob, t, ids).reshape(-1))
        out.append((ids, data))
    return out


def key_to_table_row(prob, keys):
    hcs = np.concatenate([[0], np.cumsum(prob.rows)]).astype(np.int64)
    t = np.searchsorted(hcs, keys, side="right") - 1
    return t, keys - hcs[t]


def allclose_report(got, ref, rtol, atol):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    rel = err / np.maximum(np.abs(ref), 1e-30)
    return dict(ok=not bool(bad.any()), n_bad=int(bad.sum()), n=int(err.size),
                max_abs=float(err.max()) if err.size else 0.0,
                max_rel=float(rel.max()) if rel.size else 0.0)


TOL = {"f32": (1e-5, 1e-6), "f16": (2e-3, 1e-3)}


# ---------------------------------------------------------------- device side
def device_inputs(prob, index_dtype="i32", device="cuda"):
    """Move a problem's jagged inputs to the GPU (torch tensors)."""
    import torch
    it = torch.int32 if index_dtype == "i32" else torch.int64
    d = dict(indices=torch.from_numpy(prob.indices).to(device=device, dtype=it),
             offsets=torch.from_numpy(prob.offsets).to(device=device, dtype=it),
             psw=None if prob.psw is None else torch.from_numpy(prob.psw).to(device),
             grad=torch.from_numpy(prob.grad).to(device))
    return d


def make_plan(prob, index_dtype="i32"):
    from pooling_tbe_forward_amd import tbe
    return tbe.tbe_plan_create(prob.rows, prob.dims,
                               tbe.TBE_F32 if prob.wdtype == "f32" else tbe.TBE_F16,
                               tbe.TBE_I32 if index_dtype == "i32" else tbe.TBE_I64,
                               weighted=prob.weighted)


def device_weights_from_host(packed, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(packed)).to(device)


def touched_rows(prob):
    """Sorted unique row ids read by each table."""
    out = []
    for t in range(prob.T):
        s, e = prob.offsets[t * prob.B], prob.offsets[(t + 1) * prob.B]
        out.append(np.unique(prob.indices[s:e]))
    return out


def rows_from_device(w_dev, prob, t, rows):
    """Read rows of table t from a packed device weight tensor (host numpy)."""
    import torch
    starts = dg.table_element_starts(prob)
    D = int(prob.dims[t])
    tab = w_dev[int(starts[t]):int(starts[t + 1])].view(-1, D)
    idx = torch.from_numpy(np.asarray(rows, dtype=np.int64)).to(w_dev.device)
    return tab.index_select(0, idx).cpu().numpy()
