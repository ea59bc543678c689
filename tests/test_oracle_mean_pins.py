"""Pins of the oracle's mean pooling against facts that do not come from the
oracle: the hand-worked example (tests/golden/mean_pooling_handworked.json)
and dense brute force with one-hot matrices whose entries are w_j / L_bag
(forward = A_t W_t, row gradients = A_t^T G_t), on toys with empty and
ragged bags."""
import json
import os

import numpy as np
import pytest

import oracle
from pooling_tbe_forward_amd import datagen as dg
from tests import helpers as H

HERE = os.path.join(os.path.dirname(__file__), "golden")
BASE = json.load(open(os.path.join(HERE, "handworked.json")))
MEAN = json.load(open(os.path.join(HERE, "mean_pooling_handworked.json")))


def _base(weighted, wdtype):
    g = BASE
    npdt = np.float32 if wdtype == oracle.F32 else np.float16
    packed = np.array(g["packed_weights"], npdt)
    rows, dims = np.array(g["rows"]), np.array(g["dims"], np.int32)
    return dict(T=g["T"], B=g["B"], rows=rows, dims=dims, packed=packed,
                tabs=oracle.dense_tables(packed, rows, dims),
                indices=np.array(g["indices"]), offsets=np.array(g["offsets"]),
                psw=np.array(g["per_sample_weights"], np.float32) if weighted else None,
                weighted=np.ones(g["T"], bool) if weighted else None)


@pytest.mark.parametrize("wdtype", [oracle.F32, oracle.F16])
@pytest.mark.parametrize("weighted", [False, True])
def test_handworked_mean(wdtype, weighted):
    p = _base(weighted, wdtype)
    sfx = "weighted" if weighted else "unweighted"
    out = oracle.forward(p["T"], p["B"], p["rows"], p["dims"], wdtype, p["tabs"], p["indices"],
                         p["offsets"], p["psw"], p["weighted"], pooling="mean")
    assert out.tolist() == MEAN["forward_" + sfx]
    gr, _ = oracle.backward_sgd(p["T"], p["B"], p["rows"], p["dims"], wdtype, p["tabs"],
                                p["indices"], p["offsets"], p["psw"], p["weighted"],
                                np.array(BASE["grad_output"], np.float32), BASE["lr"],
                                np.array(BASE["unique_keys"]), write_back=True, pooling="mean")
    for k, want in enumerate(MEAN["row_grads_" + sfx]):
        assert gr[k, :len(want)].tolist() == want
    assert p["packed"].astype(np.float64).tolist() == MEAN["weights_after_" + sfx]


def _onehot_mean(prob, t):
    A = np.zeros((prob.B, int(prob.rows[t])), np.float64)
    for b in range(prob.B):
        s, e = prob.offsets[t * prob.B + b], prob.offsets[t * prob.B + b + 1]
        for j in range(s, e):
            w = float(prob.psw[j]) if (prob.psw is not None and prob.weighted[t]) else 1.0
            A[b, prob.indices[j]] += w / (e - s)
    return A


@pytest.mark.parametrize("seed", [1, 2, 3])
@pytest.mark.parametrize("weighted", ["none", "all"])
def test_mean_bruteforce_onehot(seed, weighted):
    prob = dg.make_problem("toy", seed=seed, weighted=weighted, B=12)
    packed = dg.packed_weights_np(prob)
    tabs = oracle.dense_tables(packed, prob.rows, prob.dims)
    out = oracle.forward(prob.T, prob.B, prob.rows, prob.dims, H.wcode(prob), tabs, prob.indices,
                         prob.offsets, prob.psw, prob.weighted, pooling="mean")
    keys = H.oracle_sort(prob, 1 << 62)["unique_keys"]
    gr, _ = oracle.backward_sgd(prob.T, prob.B, prob.rows, prob.dims, H.wcode(prob), tabs,
                                prob.indices, prob.offsets, prob.psw, prob.weighted, prob.grad,
                                prob.lr, keys, pooling="mean")
    cols = np.concatenate([[0], np.cumsum(prob.dims)])
    W, pos = [], 0
    for t in range(prob.T):
        n = int(prob.rows[t]) * int(prob.dims[t])
        W.append(packed[pos:pos + n].astype(np.float64).reshape(int(prob.rows[t]), -1))
        pos += n
    tt, rr = H.key_to_table_row(prob, keys)
    for t in range(prob.T):
        A = _onehot_mean(prob, t)
        np.testing.assert_allclose(out[:, cols[t]:cols[t + 1]], A @ W[t], rtol=1e-13, atol=1e-15)
        Gt = A.T @ prob.grad[:, cols[t]:cols[t + 1]].astype(np.float64)
        sel = np.flatnonzero(tt == t)
        np.testing.assert_allclose(gr[sel, :int(prob.dims[t])], Gt[rr[sel]], rtol=1e-12,
                                   atol=1e-14)
    assert (prob.lengths == 0).any()      # the toy keeps an empty bag


def test_mean_adagrad_uses_mean_gradient():
    """Adagrad under mean pooling sees the mean-pooling row gradient."""
    prob = dg.make_problem("toy", seed=4, weighted="all")
    packed = dg.packed_weights_np(prob)
    keys = H.oracle_sort(prob, 1 << 62)["unique_keys"]
    tabs = oracle.dense_tables(packed.copy(), prob.rows, prob.dims)
    g_sgd, _ = oracle.backward_sgd(prob.T, prob.B, prob.rows, prob.dims, H.wcode(prob), tabs,
                                   prob.indices, prob.offsets, prob.psw, prob.weighted, prob.grad,
                                   0.0, keys, pooling="mean")
    g_ada, _, _ = oracle.backward_adagrad(prob.T, prob.B, prob.rows, prob.dims, H.wcode(prob),
                                          tabs, prob.indices, prob.offsets, prob.psw,
                                          prob.weighted, prob.grad, 0.1, 1e-8, keys,
                                          np.zeros(keys.size, np.float32), pooling="mean")
    assert np.array_equal(g_sgd, g_ada)
