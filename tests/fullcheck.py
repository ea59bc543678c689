"""Whole-output parity checks for full-size problems: every bag of the
forward and every touched row of the backward against the CPU oracle, and
every untouched row against the generator.

Work goes table by table, so the host holds one table's touched rows at a
time (regenerated with datagen.weight_rows, the generator the oracle is
pinned to), and the oracle runs on the process's host threads (its OpenMP
loops give the same bits as one thread).  Only marshalling lives here.
"""
from __future__ import annotations

import dataclasses
import os

import numpy as np

import oracle
from pooling_tbe_forward_amd import datagen as dg
from tests import helpers as H


def host_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


class _Threads:
    def __enter__(self):
        oracle.set_threads(host_threads())

    def __exit__(self, *exc):
        oracle.set_threads(1)


def _merge(reps):
    ok = all(r["ok"] for r in reps)
    return dict(ok=ok, n_bad=sum(r["n_bad"] for r in reps), n=sum(r["n"] for r in reps),
                max_abs=max((r["max_abs"] for r in reps), default=0.0),
                max_rel=max((r["max_rel"] for r in reps), default=0.0),
                bad_tables=[r["table"] for r in reps if not r["ok"]])


def table_problem(prob, t):
    """Table t of `prob` as a one-table problem: its bags, ids, per-sample
    weights and its columns of grad_output.  The operator is separable by
    table (a table's output columns and row gradients depend only on its own
    bags), so the oracle on this problem gives table t's part of the whole
    result."""
    s, e = int(prob.offsets[t * prob.B]), int(prob.offsets[(t + 1) * prob.B])
    c0 = int(prob.dims[:t].sum())
    D = int(prob.dims[t])
    return dataclasses.replace(
        prob, T=1, rows=prob.rows[t:t + 1].copy(), dims=prob.dims[t:t + 1].copy(),
        weighted=prob.weighted[t:t + 1].copy(), lengths=prob.lengths[t:t + 1].copy(),
        offsets=prob.offsets[t * prob.B:(t + 1) * prob.B + 1] - s,
        indices=prob.indices[s:e], psw=None if prob.psw is None else prob.psw[s:e],
        grad=np.ascontiguousarray(prob.grad[:, c0:c0 + D]))


def _lookups_of(prob, t):
    s, e = int(prob.offsets[t * prob.B]), int(prob.offsets[(t + 1) * prob.B])
    return prob.indices[s:e]


def _held(sub, tsrc, prob):
    """Sparse oracle table of the sub-problem: its touched rows, generated
    with the full problem's table index (the generator keys on it)."""
    rows = np.unique(sub.indices)
    data = np.ascontiguousarray(dg.weight_rows(prob, tsrc, rows).reshape(-1))
    return rows, [(rows, data)]


def forward_all(prob, out, pooling="sum", tol=None):
    """Every element of the [B, sum D] output `out` (host array) against the
    oracle's fp64 pooled sums, within the weight dtype's tolerance (or tol =
    (rtol, atol))."""
    rtol, atol = tol or H.TOL[prob.wdtype]
    cols = np.concatenate([[0], np.cumsum(prob.dims)]).astype(np.int64)
    reps = []
    with _Threads():
        for t in range(prob.T):
            D = int(prob.dims[t])
            sub = table_problem(prob, t)
            _, tabs = _held(sub, t, prob)
            ref = oracle.forward(1, sub.B, sub.rows, sub.dims, H.wcode(sub), tabs, sub.indices,
                                 sub.offsets, sub.psw, sub.weighted, pooling=pooling)
            rep = H.allclose_report(out[:, cols[t]:cols[t] + D], ref, rtol, atol)
            rep["table"] = t
            reps.append(rep)
    return _merge(reps)


def backward_all(prob, w_dev, pooling="sum", adagrad=None):
    """Every touched row of the updated device weights against the oracle.

    adagrad: None for SGD, else (state0 host fp32 [sum rows], s_dev device
    state after the step, eps); the new state of every touched row is
    checked too."""
    rtol, atol = H.TOL[prob.wdtype]
    hcs = np.concatenate([[0], np.cumsum(prob.rows)]).astype(np.int64)
    reps = []
    s_all = adagrad[1].cpu().numpy() if adagrad else None
    with _Threads():
        for t in range(prob.T):
            D = int(prob.dims[t])
            sub = table_problem(prob, t)
            rows, tabs = _held(sub, t, prob)
            if rows.size == 0:
                continue
            args = (1, sub.B, sub.rows, sub.dims, H.wcode(sub), tabs, sub.indices, sub.offsets,
                    sub.psw, sub.weighted, sub.grad, sub.lr)
            if adagrad:
                state0, _, eps = adagrad
                _, nr, st = oracle.backward_adagrad(*args, eps, rows, state0[hcs[t] + rows],
                                                    pooling=pooling)
                srep = H.allclose_report(s_all[hcs[t] + rows], st, rtol, atol)
                srep["table"] = t
                reps.append(srep)
            else:
                _, nr = oracle.backward_sgd(*args, rows, pooling=pooling)
            got = H.rows_from_device(w_dev, prob, t, rows).astype(np.float64)
            rep = H.allclose_report(got, nr, rtol, atol)
            rep["table"] = t
            reps.append(rep)
    return _merge(reps)


def untouched_all(prob, w_dev, state=None):
    """Every row no lookup read keeps the generator's bits: on the device,
    each table is compared with a freshly generated copy, and every row that
    differs must be one the batch read.  state: optional (state0 host, s_dev)
    for row-wise Adagrad, whose untouched entries must keep their bits."""
    import torch
    starts = dg.table_element_starts(prob)
    hcs = np.concatenate([[0], np.cumsum(prob.rows)]).astype(np.int64)
    dt = torch.float32 if prob.wdtype == "f32" else torch.float16
    it = torch.int32 if prob.wdtype == "f32" else torch.int16
    for t in range(prob.T):
        D = int(prob.dims[t])
        fresh = torch.empty(int(prob.rows[t]) * D, dtype=dt, device=w_dev.device)
        dg.table_weights_torch(prob, t, fresh)
        cur = w_dev[int(starts[t]):int(starts[t + 1])]
        differ = (cur.view(it) != fresh.view(it)).view(-1, D).any(dim=1)
        changed = torch.nonzero(differ).view(-1).cpu().numpy()
        del fresh, differ
        touched = np.unique(_lookups_of(prob, t))
        stray = np.setdiff1d(changed, touched)
        assert stray.size == 0, (t, stray[:8])
        if state is not None:
            state0, s_dev = state
            lo, hi = int(hcs[t]), int(hcs[t + 1])
            s_now = s_dev[lo:hi].cpu().numpy()
            keep = np.ones(hi - lo, bool)
            keep[touched] = False
            assert np.array_equal(s_now[keep].view(np.uint32), state0[lo:hi][keep].view(np.uint32)), t
