"""GPU parity of mean pooling (tbe_plan_set_pooling(plan, "mean")) through the
C ABI against the oracle: forward (empty bags stay zero), backward-SGD and
row-wise Adagrad (each lookup's contribution divided by its bag's length),
prepare/apply, and the error code of an unknown mode."""
import numpy as np
import pytest
import torch

import oracle
from pooling_tbe_forward_amd import datagen as dg
from pooling_tbe_forward_amd import tbe
from tests import fullcheck
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _plan(prob):
    plan = H.make_plan(prob)
    tbe.tbe_plan_set_pooling(plan, "mean")
    return plan


@pytest.mark.parametrize("name,B", [("toy", None), ("uniform", 256), ("mixed", 64),
                                    ("hist", 64), ("stress", 128)])
def test_mean_forward_vs_oracle(name, B):
    prob = dg.make_problem(name, seed=900, **({} if B is None else dict(B=B)))
    w = dg.packed_weights_torch(prob, "cuda")
    plan = _plan(prob)
    d = H.device_inputs(prob)
    out = torch.full((prob.B, prob.sum_D), float("nan"), dtype=torch.float32, device="cuda")
    tbe.tbe_forward(plan, prob.B, w, d["indices"], d["offsets"], d["psw"], out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    # every bag; fp32 accumulation of exact fp16 values stays inside the fp32 bound
    rep = fullcheck.forward_all(prob, got, pooling="mean", tol=(1e-5, 1e-6))
    assert rep["ok"], rep
    cols = np.concatenate([[0], np.cumsum(prob.dims)])
    if name == "toy":
        assert np.all(got[2, cols[1]:cols[2]] == 0)     # the forced empty bag (t=1, b=2)



@pytest.mark.parametrize("seed,max_len", [(71, 90), (72, 2600)])
def test_mean_histogram_path_bit_exact(seed, max_len):
    """Mean pooling on the histogram path: small fp16 tables with integer
    weights, so every bag's sum is exact on both forward paths and the one
    division per bag gives the same bits; both equal the fp64 quotient to an
    ulp.  max_len 2600 makes bags longer than one 2048-id counting window."""
    prob, packed = dg.exact_problem(seed, T=3, B=45, dims=(64, 128, 16), wdtype="f16",
                                    weighted=False, max_len=max_len, max_rows=40)
    # empty bags (one per table) must stay zero on both paths
    keep = np.ones(prob.indices.size, bool)
    for t in range(prob.T):
        g = t * prob.B + 3 + t
        keep[prob.offsets[g]:prob.offsets[g + 1]] = False
        prob.lengths[t, 3 + t] = 0
    prob.indices = prob.indices[keep]
    prob.offsets = np.concatenate([[0], np.cumsum(prob.lengths.ravel())]).astype(np.int64)
    w = H.device_weights_from_host(packed)
    outs = []
    for mode in (2, 1):   # histogram path forced, then the gather alone
        plan = _plan(prob)
        tbe.tbe_set_tuning(plan, hist_mode=mode)
        d = H.device_inputs(prob)
        out = torch.full((prob.B, prob.sum_D), float("nan"), dtype=torch.float32, device="cuda")
        tbe.tbe_forward(plan, prob.B, w, d["indices"], d["offsets"], d["psw"], out)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    tabs = oracle.dense_tables(packed, prob.rows, prob.dims)
    ref = oracle.forward(prob.T, prob.B, prob.rows, prob.dims, H.wcode(prob), tabs, prob.indices,
                         prob.offsets, prob.psw, prob.weighted, pooling="mean")
    rep = H.allclose_report(outs[0], ref, 1e-6, 0.0)
    assert rep["ok"], rep
    assert (prob.lengths == 0).any()


def _oracle_rows(prob, keys, pooling, state_in=None, eps=None):
    tt, rr = H.key_to_table_row(prob, keys)
    tabs = H.sparse_tables(prob, [np.unique(rr[tt == t]) for t in range(prob.T)])
    if state_in is None:
        return oracle.backward_sgd(prob.T, prob.B, prob.rows, prob.dims, H.wcode(prob), tabs,
                                   prob.indices, prob.offsets, prob.psw, prob.weighted, prob.grad,
                                   prob.lr, keys, pooling=pooling)[1], None
    _, nr, st = oracle.backward_adagrad(prob.T, prob.B, prob.rows, prob.dims, H.wcode(prob),
                                        tabs, prob.indices, prob.offsets, prob.psw,
                                        prob.weighted, prob.grad, prob.lr, eps, keys,
                                        state_in[keys], pooling=pooling)
    return nr, st


def _rows_on_device(prob, w_dev, keys, like):
    tt, rr = H.key_to_table_row(prob, keys)
    got = np.array(like)
    for t in range(prob.T):
        sel = np.flatnonzero(tt == t)
        if sel.size:
            got[sel, :int(prob.dims[t])] = H.rows_from_device(w_dev, prob, t, rr[sel])
    return got


@pytest.mark.parametrize("name,B,tau", [("toy", None, 2), ("uniform", 256, 128),
                                        ("stress", 256, 16), ("mixed", 64, 128)])
@pytest.mark.parametrize("opt", ["sgd", "adagrad"])
@pytest.mark.parametrize("sort_mode", [1, 2])
def test_mean_backward_vs_oracle(name, B, tau, opt, sort_mode):
    prob = dg.make_problem(name, seed=910, **({} if B is None else dict(B=B)))
    plan = _plan(prob)
    tbe.tbe_set_tuning(plan, tau=tau, chunk=8, sort_mode=sort_mode)
    d = H.device_inputs(prob)
    w = dg.packed_weights_torch(prob, "cuda")
    ws = tbe.alloc_workspace(plan, prob.B, prob.N)
    state0 = np.random.default_rng(1).random(int(np.sum(prob.rows)), dtype=np.float32)
    s_dev = torch.from_numpy(state0.copy()).cuda()
    if opt == "sgd":
        tbe.tbe_backward_sgd(plan, prob.B, w, d["indices"], d["offsets"], d["psw"], d["grad"],
                             prob.lr, ws)
    else:
        tbe.tbe_backward_adagrad(plan, prob.B, w, s_dev, d["indices"], d["offsets"], d["psw"],
                                 d["grad"], prob.lr, ws)
    torch.cuda.synchronize()
    rep = fullcheck.backward_all(prob, w, pooling="mean",
                                 adagrad=(state0, s_dev, tbe.ADAGRAD_EPS) if opt == "adagrad"
                                 else None)
    assert rep["ok"], rep
    fullcheck.untouched_all(prob, w, state=(state0, s_dev))
    keys = H.oracle_sort(prob, tau)["unique_keys"]
    nr, _ = _oracle_rows(prob, keys[:50], "mean")
    # mean and sum differ wherever a bag has more than one lookup
    if name == "uniform":
        nr_sum, _ = _oracle_rows(prob, keys[:50], "sum")
        assert not np.allclose(nr_sum, nr[:50])


def test_mean_prepare_apply_matches_whole():
    prob = dg.make_problem("stress", seed=920, B=256)
    plan = _plan(prob)
    d = H.device_inputs(prob)
    w1 = dg.packed_weights_torch(prob, "cuda")
    ws = tbe.alloc_workspace(plan, prob.B, prob.N)
    tbe.tbe_backward_sgd(plan, prob.B, w1, d["indices"], d["offsets"], d["psw"], d["grad"],
                         prob.lr, ws)
    w2 = dg.packed_weights_torch(prob, "cuda")
    tbe.tbe_backward_prepare(plan, prob.B, d["indices"], d["offsets"], d["psw"], ws)
    tbe.tbe_backward_apply(plan, prob.B, prob.N, d["psw"] is not None, w2, d["grad"], prob.lr, ws)
    torch.cuda.synchronize()
    assert torch.equal(w1.view(torch.int32), w2.view(torch.int32))
    rep = fullcheck.backward_all(prob, w2, pooling="mean")
    assert rep["ok"], rep
    fullcheck.untouched_all(prob, w2)


def test_pooling_mode_errors():
    prob = dg.make_problem("toy", seed=1)
    plan = H.make_plan(prob)
    assert tbe.lib().tbe_plan_set_pooling(plan.handle, 2) == tbe.TBE_EINVAL
    assert tbe.lib().tbe_plan_set_pooling(plan.handle, -1) == tbe.TBE_EINVAL
    tbe.tbe_plan_set_pooling(plan, "mean")
    tbe.tbe_plan_set_pooling(plan, "sum")
