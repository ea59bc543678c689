"""Seeded randomized parity sweep through the C ABI.

Each case is an exact-arithmetic problem (integer weights in [-8, 8],
per-sample weights in {0.25, 0.5, 1, 2}, integer output gradients, lr = 0.5):
every summation order yields the same bits, so forward, integer stage and
backward-SGD must equal the oracle exactly, whatever table count, widths
(including widths that are not a multiple of 4 and widths above 256), index
type, weight type, run threshold, chunk size or forward path the case draws.
"""
import numpy as np
import pytest
import torch

from pooling_tbe_forward_amd import datagen as dg
from pooling_tbe_forward_amd import tbe
from tests import helpers as H

pytestmark = pytest.mark.gpu

_DIMS = [1, 2, 3, 4, 5, 8, 12, 16, 24, 32, 64, 100, 128, 256, 300, 520]


def _cases(n=64, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        T = int(rng.integers(1, 6))
        out.append(dict(
            seed=1000 + k, T=T, B=int(rng.integers(1, 200)),
            dims=tuple(int(x) for x in rng.choice(_DIMS, size=T)),
            wdtype=str(rng.choice(["f32", "f16"])), weighted=bool(rng.integers(0, 2)),
            index_dtype=str(rng.choice(["i32", "i64"])),
            max_len=int(rng.choice([3, 12, 40, 90])), max_rows=int(rng.choice([5, 40, 300])),
            tau=int(rng.choice([1, 2, 8, 64, 2 ** 31 - 1])),
            chunk=int(rng.choice([1, 3, 16, 256])),
            hist_mode=int(rng.choice([0, 1, 2])), sort_mode=int(rng.choice([0, 1, 2]))))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[f"case{k}" for k in range(len(CASES))])
def test_random_exact_case(case):
    c = dict(case)
    prob, packed = dg.exact_problem(c["seed"], T=c["T"], B=c["B"], dims=c["dims"],
                                    wdtype=c["wdtype"], weighted=c["weighted"],
                                    max_len=c["max_len"], max_rows=c["max_rows"])
    plan = H.make_plan(prob, c["index_dtype"])
    tbe.tbe_set_tuning(plan, tau=c["tau"], chunk=c["chunk"], hist_mode=c["hist_mode"],
                       sort_mode=c["sort_mode"])
    d = H.device_inputs(prob, c["index_dtype"])
    w = H.device_weights_from_host(packed)

    # forward
    out = torch.full((prob.B, prob.sum_D), float("nan"), device="cuda")
    tbe.tbe_forward(plan, prob.B, w, d["indices"], d["offsets"], d["psw"], out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.float64), H.oracle_forward(prob, packed)), c

    # integer stage
    ws = tbe.alloc_workspace(plan, prob.B, prob.N)
    if prob.N:
        v = tbe.tbe_sort_rle(plan, prob.B, d["indices"], d["offsets"], ws)
        torch.cuda.synchronize()
        u32 = lambda t: t.cpu().numpy().view(np.uint32).astype(np.int64)
        cnt = u32(v["counts"])
        o = H.oracle_sort(prob, c["tau"])
        assert cnt[4] == 0 and int(cnt[0]) == o["num_runs"], c
        assert np.array_equal(u32(v["sorted_pos"]), o["sorted_pos"]), c
        R, L = int(cnt[0]), int(cnt[2])
        assert np.array_equal(u32(v["run_len"][:R]), o["run_len"]), c
        assert np.array_equal(u32(v["long_runs"][:L]), o["long_runs"]), c

    # backward + SGD (the same workspace: the sort left its control block clean)
    tbe.tbe_backward_sgd(plan, prob.B, w, d["indices"], d["offsets"], d["psw"], d["grad"],
                         prob.lr, ws)
    torch.cuda.synchronize()
    ref = packed.copy()
    H.oracle_backward(prob, ref)
    assert np.array_equal(w.cpu().numpy().view(np.uint8), ref.view(np.uint8)), c


def test_random_exact_bulk():
    """Two thousand more small cases in one test (another seed), failing on the
    first mismatch with its case."""
    for c in _cases(n=2000, seed=11):
        test_random_exact_case(c)


def test_random_exact_larger_batches():
    """Batches of 200-3000 samples, so tables span several radix tiles (and the
    per-table sort its several tiles per table), up to 5000 rows per table."""
    rng = np.random.default_rng(13)
    for k in range(60):
        T = int(rng.integers(1, 9))
        test_random_exact_case(dict(
            seed=5000 + k, T=T, B=int(rng.integers(200, 3000)),
            dims=tuple(int(x) for x in rng.choice(_DIMS[:12], size=T)),
            wdtype=str(rng.choice(["f32", "f16"])), weighted=bool(rng.integers(0, 2)),
            index_dtype=str(rng.choice(["i32", "i64"])),
            max_len=int(rng.choice([3, 12, 40, 90])),
            max_rows=int(rng.choice([5, 40, 300, 5000])),
            tau=int(rng.choice([1, 8, 64, 2 ** 31 - 1])), chunk=int(rng.choice([3, 16, 256])),
            hist_mode=int(rng.choice([0, 1, 2])), sort_mode=int(rng.choice([0, 1, 2]))))
