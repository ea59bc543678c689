"""GPU parity of the backward with exact row-wise Adagrad, through the C ABI,
against the CPU oracle (oracle_backward_adagrad): updated rows within the
weight dtype's tolerance of the fp64 oracle, the new row state within the
same tolerance of the oracle's fp32 state, untouched rows and states
bit-identical; the hand-worked case (every value exact) bit-exact for every
short / long split."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from pooling_tbe_forward_amd import datagen as dg
from pooling_tbe_forward_amd import tbe
from tests import helpers as H
from tests import fullcheck
from tests.test_gpu_backward import _gold_problem

pytestmark = pytest.mark.gpu
AGOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "adagrad_handworked.json")))


def _state0(prob, seed, scale=1.0):
    """A seeded initial row state (fp32, one value per row of every table)."""
    rng = np.random.default_rng(seed)
    return (rng.random(int(np.sum(prob.rows)), dtype=np.float32) * scale).astype(np.float32)


def gpu_adagrad(prob, w_dev, state_dev, lr=None, eps=tbe.ADAGRAD_EPS, plan=None, **tuning):
    plan = plan or H.make_plan(prob)
    if tuning:
        tbe.tbe_set_tuning(plan, **tuning)
    d = H.device_inputs(prob)
    ws = tbe.alloc_workspace(plan, prob.B, prob.N)
    tbe.tbe_backward_adagrad(plan, prob.B, w_dev, state_dev, d["indices"], d["offsets"],
                             d["psw"], d["grad"], prob.lr if lr is None else lr, ws, eps=eps)
    torch.cuda.synchronize()
    return w_dev, state_dev


def _oracle_sampled(prob, keys, state_in, eps, tables=None):
    """Oracle Adagrad rows for `keys` (rows generated on the host)."""
    tt, rr = H.key_to_table_row(prob, keys)
    if tables is None:
        tables = H.sparse_tables(prob, [np.unique(rr[tt == t]) for t in range(prob.T)])
    return oracle.backward_adagrad(prob.T, prob.B, prob.rows, prob.dims, H.wcode(prob), tables,
                                   prob.indices, prob.offsets, prob.psw, prob.weighted,
                                   prob.grad, prob.lr, eps, keys, state_in[keys])


def _check_sampled(prob, w_dev, s_dev, keys, state0, eps):
    _, nr, st = _oracle_sampled(prob, keys, state0, eps)
    tt, rr = H.key_to_table_row(prob, keys)
    got = np.zeros_like(nr)
    for t in range(prob.T):
        sel = np.flatnonzero(tt == t)
        if sel.size:
            D = int(prob.dims[t])
            got[sel, :D] = H.rows_from_device(w_dev, prob, t, rr[sel]).astype(np.float64)
            got[sel, D:] = nr[sel, D:]
    rtol, atol = H.TOL[prob.wdtype]
    rep = H.allclose_report(got, nr, rtol, atol)
    assert rep["ok"], ("rows", rep)
    s_got = s_dev.cpu().numpy()[keys]
    rep = H.allclose_report(s_got, st, rtol, atol)
    assert rep["ok"], ("state", rep)


def _untouched(prob, w_dev, s_dev, state0, unique_keys, n=2000, seed=3):
    rng = np.random.default_rng(seed)
    hcs = np.concatenate([[0], np.cumsum(prob.rows)])
    cand = np.setdiff1d(rng.integers(0, int(hcs[-1]), size=2 * n), unique_keys)[:n]
    assert np.array_equal(s_dev.cpu().numpy()[cand].view(np.uint32), state0[cand].view(np.uint32))
    tt, rr = H.key_to_table_row(prob, cand)
    for t in range(prob.T):
        sel = rr[tt == t]
        if sel.size:
            got = H.rows_from_device(w_dev, prob, t, sel)
            want = dg.weight_rows(prob, t, sel)
            u = np.uint16 if got.dtype == np.float16 else np.uint32
            assert np.array_equal(got.view(u), want.view(u))


@pytest.mark.parametrize("wdtype", ["f32", "f16"])
@pytest.mark.parametrize("weighted", [False, True])
@pytest.mark.parametrize("tau,chunk", [(2 ** 31 - 1, 256), (2, 1), (1, 1), (1, 3)])
def test_handworked_adagrad_bit_exact(wdtype, weighted, tau, chunk):
    prob, packed = _gold_problem(weighted, wdtype)
    case = AGOLD["weighted" if weighted else "unweighted"]
    state = torch.tensor(case["state_in"], dtype=torch.float32, device="cuda")  # keys 0..4
    w, s = gpu_adagrad(prob, H.device_weights_from_host(packed), state, eps=AGOLD["eps"],
                       tau=tau, chunk=chunk)
    assert w.cpu().numpy().astype(np.float64).tolist() == case["weights_after"]
    assert s.cpu().numpy().astype(np.float64).tolist() == case["state_out"]


@pytest.mark.parametrize("seed", [1, 2, 3])
@pytest.mark.parametrize("weighted", ["none", "all"])
@pytest.mark.parametrize("tau", [256, 2])
def test_toy_adagrad_vs_oracle(seed, weighted, tau):
    prob = dg.make_problem("toy", seed=seed, weighted=weighted)
    packed = dg.packed_weights_np(prob)
    state0 = _state0(prob, seed)
    w, s = gpu_adagrad(prob, H.device_weights_from_host(packed),
                       torch.from_numpy(state0.copy()).cuda(), tau=tau, chunk=1)
    keys = H.oracle_sort(prob, 1 << 62)["unique_keys"]
    tabs = oracle.dense_tables(packed.copy(), prob.rows, prob.dims)
    _, nr, st = _oracle_sampled(prob, keys, state0, tbe.ADAGRAD_EPS, tables=tabs)
    w_after = w.cpu().numpy()
    wo, _, _ = oracle.layout(prob.rows, prob.dims)
    tt, rr = H.key_to_table_row(prob, keys)
    touched = np.zeros(w_after.size, bool)
    got = np.zeros_like(nr)
    for k in range(keys.size):
        D = int(prob.dims[tt[k]])
        a = int(wo[tt[k]]) + int(rr[k]) * D
        touched[a:a + D] = True
        got[k, :D] = w_after[a:a + D]
        got[k, D:] = nr[k, D:]
    assert H.allclose_report(got, nr, *H.TOL[prob.wdtype])["ok"]
    assert H.allclose_report(s.cpu().numpy()[keys], st, *H.TOL[prob.wdtype])["ok"]
    assert np.array_equal(w_after[~touched].view(np.uint32), packed[~touched].view(np.uint32))
    keep = np.setdiff1d(np.arange(state0.size), keys)
    assert np.array_equal(s.cpu().numpy()[keep], state0[keep])


@pytest.mark.parametrize("name,B,tau", [("uniform", 256, 256), ("stress", 256, 16),
                                        ("mixed", 64, 256), ("hist", 64, 256),
                                        ("band", 512, 64)])
def test_reduced_adagrad_vs_oracle(name, B, tau):
    prob = dg.make_problem(name, seed=700 + B, B=B)
    state0 = _state0(prob, 7, scale=0.5)
    w_dev = dg.packed_weights_torch(prob, "cuda")
    s_dev = torch.from_numpy(state0.copy()).cuda()
    gpu_adagrad(prob, w_dev, s_dev, tau=tau)
    rep = fullcheck.backward_all(prob, w_dev, adagrad=(state0, s_dev, tbe.ADAGRAD_EPS))
    assert rep["ok"], rep
    fullcheck.untouched_all(prob, w_dev, state=(state0, s_dev))


@pytest.mark.parametrize("name", ["stress", "uniform", "mixed", "band"])
def test_full_size_adagrad_every_row(name):
    """Full configuration at the plan's default tuning: every touched row and
    its state against the oracle, every other row and state unchanged."""
    prob = dg.make_problem(name)
    state0 = _state0(prob, 9)
    w_dev = dg.packed_weights_torch(prob, "cuda")
    s_dev = torch.from_numpy(state0.copy()).cuda()
    gpu_adagrad(prob, w_dev, s_dev)
    rep = fullcheck.backward_all(prob, w_dev, adagrad=(state0, s_dev, tbe.ADAGRAD_EPS))
    assert rep["ok"], rep
    fullcheck.untouched_all(prob, w_dev, state=(state0, s_dev))
    del w_dev, s_dev
    torch.cuda.empty_cache()


def test_two_steps_carry_the_state():
    prob = dg.make_problem("stress", seed=41, B=128)
    state0 = np.zeros(int(np.sum(prob.rows)), np.float32)
    w_dev = dg.packed_weights_torch(prob, "cuda")
    s_dev = torch.zeros(state0.size, dtype=torch.float32, device="cuda")
    plan = H.make_plan(prob)
    tbe.tbe_set_tuning(plan, tau=16, chunk=8)
    for _ in range(2):
        gpu_adagrad(prob, w_dev, s_dev, plan=plan)
    keys = H.oracle_sort(prob, 1 << 62)["unique_keys"]
    tt, rr = H.key_to_table_row(prob, keys)
    tabs = H.sparse_tables(prob, [np.unique(rr[tt == t]) for t in range(prob.T)])
    s1 = oracle.backward_adagrad(prob.T, prob.B, prob.rows, prob.dims, H.wcode(prob), tabs,
                                 prob.indices, prob.offsets, prob.psw, prob.weighted, prob.grad,
                                 prob.lr, tbe.ADAGRAD_EPS, keys, state0[keys], write_back=True)[2]
    _, nr, s2 = oracle.backward_adagrad(prob.T, prob.B, prob.rows, prob.dims, H.wcode(prob), tabs,
                                        prob.indices, prob.offsets, prob.psw, prob.weighted,
                                        prob.grad, prob.lr, tbe.ADAGRAD_EPS, keys, s1)
    got = np.zeros_like(nr)
    for t in range(prob.T):
        sel = np.flatnonzero(tt == t)
        got[sel, :int(prob.dims[t])] = H.rows_from_device(w_dev, prob, t, rr[sel])
    assert H.allclose_report(got, nr, *H.TOL["f32"])["ok"]
    assert H.allclose_report(s_dev.cpu().numpy()[keys], s2, *H.TOL["f32"])["ok"]


def test_prepare_apply_adagrad_matches_whole():
    prob = dg.make_problem("mixed", seed=43, B=64)
    state0 = _state0(prob, 4)
    plan = H.make_plan(prob)
    d = H.device_inputs(prob)
    w1 = dg.packed_weights_torch(prob, "cuda")
    s1 = torch.from_numpy(state0.copy()).cuda()
    gpu_adagrad(prob, w1, s1, plan=plan)
    w2 = dg.packed_weights_torch(prob, "cuda")
    s2 = torch.from_numpy(state0.copy()).cuda()
    ws = tbe.alloc_workspace(plan, prob.B, prob.N)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    tbe.tbe_backward_prepare(plan, prob.B, d["indices"], d["offsets"], d["psw"], ws, stream=side)
    ev = torch.cuda.Event()
    ev.record(side)
    torch.cuda.current_stream().wait_event(ev)
    tbe.tbe_backward_apply_adagrad(plan, prob.B, prob.N, d["psw"] is not None, w2, s2, d["grad"],
                                   prob.lr, ws)
    torch.cuda.synchronize()
    assert torch.equal(w1.view(torch.int16), w2.view(torch.int16))
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    rep = fullcheck.backward_all(prob, w2, adagrad=(state0, s2, tbe.ADAGRAD_EPS))
    assert rep["ok"], rep
    fullcheck.untouched_all(prob, w2, state=(state0, s2))


def test_adagrad_deterministic_and_lr_zero():
    prob = dg.make_problem("stress", seed=44, B=512)
    state0 = _state0(prob, 5)
    outs = []
    for lr in (prob.lr, prob.lr, 0.0):
        w = dg.packed_weights_torch(prob, "cuda")
        s = torch.from_numpy(state0.copy()).cuda()
        gpu_adagrad(prob, w, s, lr=lr, tau=32, chunk=16)
        outs.append((w, s))
    assert torch.equal(outs[0][0].view(torch.int32), outs[1][0].view(torch.int32))
    assert torch.equal(outs[0][1].view(torch.int32), outs[1][1].view(torch.int32))
    w0 = dg.packed_weights_torch(prob, "cuda")
    assert torch.equal(outs[2][0].view(torch.int32), w0.view(torch.int32))   # lr = 0
    assert torch.equal(outs[2][1].view(torch.int32), outs[0][1].view(torch.int32))


def test_adagrad_errors():
    prob = dg.make_problem("toy", seed=1)
    plan = H.make_plan(prob)
    d = H.device_inputs(prob)
    ws = tbe.alloc_workspace(plan, prob.B, prob.N)
    w = dg.packed_weights_torch(prob, "cuda")
    s = torch.zeros(int(np.sum(prob.rows)) + 1, dtype=torch.float32, device="cuda")
    L = tbe.lib()
    args = lambda st, eps: (plan.handle, prob.B, tbe._ptr(w), st, tbe._ptr(d["indices"]),
                            prob.N, tbe._ptr(d["offsets"]), None, tbe._ptr(d["grad"]), 0.1, eps,
                            tbe._ptr(ws), ws.numel(), None)
    assert L.tbe_backward_adagrad(*args(None, 1e-8)) == tbe.TBE_EINVAL
    import ctypes
    mis = ctypes.c_void_p(s.data_ptr() + 2)
    assert L.tbe_backward_adagrad(*args(mis, 1e-8)) == tbe.TBE_EINVAL
    assert L.tbe_backward_adagrad(*args(tbe._ptr(s), -1.0)) == tbe.TBE_EINVAL
    assert L.tbe_backward_adagrad(*args(tbe._ptr(s), float("nan"))) == tbe.TBE_EINVAL
    torch.cuda.synchronize()
    assert torch.equal(w, dg.packed_weights_torch(prob, "cuda"))
    # a row wider than one worker: D = 512 fp32 needs 128 lanes of 4
    wide = tbe.tbe_plan_create([16], [512], 0, 0)
    wd = torch.zeros(16 * 512, dtype=torch.float32, device="cuda")
    ix = torch.zeros(4, dtype=torch.int32, device="cuda")
    of = torch.tensor([0, 4], dtype=torch.int32, device="cuda")
    g = torch.zeros(1, 512, dtype=torch.float32, device="cuda")
    sw = torch.zeros(16, dtype=torch.float32, device="cuda")
    wsw = tbe.alloc_workspace(wide, 1, 4)
    with pytest.raises(tbe.TBEError) as e:
        tbe.tbe_backward_adagrad(wide, 1, wd, sw, ix, of, None, g, 0.1, wsw)
    assert e.value.status == tbe.TBE_ENOTSUP
    # D = 256 fp32 fits (64 lanes of 4)
    ok = tbe.tbe_plan_create([16], [256], 0, 0)
    wo = torch.zeros(16 * 256, dtype=torch.float32, device="cuda")
    g2 = torch.ones(1, 256, dtype=torch.float32, device="cuda")
    wso = tbe.alloc_workspace(ok, 1, 4)
    tbe.tbe_backward_adagrad(ok, 1, wo, sw, ix, of, None, g2, 0.5, wso, eps=0.0)
    torch.cuda.synchronize()
    # row 0 read 4 times: g = 4 everywhere, mean square 16, state 16, step 0.5/4*4 = 0.5
    assert sw[0].item() == 16.0
    assert torch.all(wo[:256] == -0.5) and torch.all(wo[256:] == 0)
