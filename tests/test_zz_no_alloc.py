"""tbe_backward_sgd_noalloc (the backward with the library's own per-GPU
workspace array) against tbe_backward_sgd on the same inputs, through the C
ABI: two calls in a row, the second on a smaller batch, each bit-identical to
the workspace entry point (the same kernels in the same order), plus the
size limit and the error word."""
import numpy as np
import pytest
import torch

from pooling_tbe_forward_amd import datagen as dg
from pooling_tbe_forward_amd import tbe
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _both(prob, tau=None):
    """Weights after tbe_backward_sgd and after tbe_backward_sgd_noalloc."""
    plan = H.make_plan(prob)
    if tau:
        tbe.tbe_set_tuning(plan, tau=tau, chunk=16)
    d = H.device_inputs(prob)
    w0 = dg.packed_weights_torch(prob, "cuda")
    w_ref, w_new = w0.clone(), w0.clone()
    ws = tbe.alloc_workspace(plan, prob.B, prob.N)
    tbe.tbe_backward_sgd(plan, prob.B, w_ref, d["indices"], d["offsets"], d["psw"], d["grad"],
                         prob.lr, ws)
    err = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    tbe.tbe_backward_sgd_noalloc(plan, prob.B, w_new, d["indices"], d["offsets"], d["psw"],
                                 d["grad"], prob.lr, error_word=err)
    torch.cuda.synchronize()
    return w0, w_ref, w_new, int(err.item())


@pytest.mark.parametrize("first,second", [
    (("stress", dict(B=512, seed=3), 16), ("stress", dict(B=96, seed=4), None)),
    (("uniform", dict(B=512, seed=5, T=4), None), ("mixed", dict(B=48, seed=6), 32)),
])
def test_noalloc_matches_workspace_entry_point(first, second):
    for name, kw, tau in (first, second):      # the second call is the smaller one
        prob = dg.make_problem(name, **kw)
        w0, w_ref, w_new, err = _both(prob, tau)
        assert err == 0
        assert not torch.equal(w_ref, w0)          # the step changed something
        assert torch.equal(w_new.view(torch.int16 if w_new.dtype == torch.float16 else torch.int32),
                           w_ref.view(torch.int16 if w_ref.dtype == torch.float16 else torch.int32))


def test_noalloc_against_oracle_toy():
    prob = dg.make_problem("toy", weighted="all")
    packed = dg.packed_weights_np(prob)
    plan = H.make_plan(prob)
    d = H.device_inputs(prob)
    w = H.device_weights_from_host(packed)
    tbe.tbe_backward_sgd_noalloc(plan, prob.B, w, d["indices"], d["offsets"], d["psw"], d["grad"],
                                 prob.lr)
    torch.cuda.synchronize()
    after = packed.copy()
    H.oracle_backward(prob, after)
    rep = H.allclose_report(w.cpu().numpy(), after.astype(np.float64), *H.TOL["f32"])
    assert rep["ok"], rep


def test_noalloc_limit_and_empty_batch():
    prob = dg.make_problem("stress", seed=7)          # 1.6M lookups: more than the array holds
    plan = H.make_plan(prob)
    assert tbe.tbe_backward_workspace_bytes(plan, prob.B, prob.N) > \
        tbe.tbe_backward_noalloc_max_bytes()
    d = H.device_inputs(prob)
    w = torch.zeros(plan.weight_elems, device="cuda")
    with pytest.raises(tbe.TBEError) as e:
        tbe.tbe_backward_sgd_noalloc(plan, prob.B, w, d["indices"], d["offsets"], d["psw"],
                                     d["grad"], prob.lr)
    assert e.value.status == tbe.TBE_ERANGE
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(w).item()) == 0
    # an empty batch updates nothing and still reports a clear error word
    empty = dg.make_problem("toy", seed=8)
    plan = H.make_plan(empty)
    w = dg.packed_weights_torch(empty, "cuda")
    w0 = w.clone()
    err = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    tbe.tbe_backward_sgd_noalloc(plan, empty.B, w, torch.zeros(0, dtype=torch.int32, device="cuda"),
                                 torch.zeros(empty.T * empty.B + 1, dtype=torch.int32,
                                             device="cuda"),
                                 None, torch.zeros(empty.B, empty.sum_D, device="cuda"), 0.1,
                                 error_word=err)
    torch.cuda.synchronize()
    assert torch.equal(w, w0) and int(err.item()) == 0
