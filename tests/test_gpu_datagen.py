"""The device half of the seeded weight generator (libtbe_datagen.so, one
launch per table) gives the host generator's bits: fp32 and fp16 tables,
both value laws, and rows across every table of the mixed workload."""
import numpy as np
import pytest

from pooling_tbe_forward_amd import datagen as dg
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _bits(a):
    return a.view(np.uint16 if a.dtype == np.float16 else np.uint32)


@pytest.mark.parametrize("name,kw", [("toy", {}), ("hist", dict(B=4)),
                                     ("mixed", dict(B=4, rows_cap=200_000)),
                                     ("uniform", dict(B=4, T=2))])
def test_device_tables_equal_host_rows(name, kw):
    prob = dg.make_problem(name, **kw)
    w = dg.packed_weights_torch(prob, "cuda")
    rng = np.random.default_rng(3)
    for t in range(prob.T):
        R = int(prob.rows[t])
        rows = np.unique(np.concatenate([[0, R - 1], rng.integers(0, R, size=300)]))
        got = H.rows_from_device(w, prob, t, rows)
        want = dg.weight_rows(prob, t, rows)
        assert np.array_equal(_bits(got), _bits(want)), (name, t)


def test_whole_small_table_and_subnormals():
    """Every element of the toy and hist tables; the fp16 tables of
    standard deviation 0.01 hold subnormals, which must survive too."""
    for name in ("toy", "hist"):
        prob = dg.make_problem(name)
        got = dg.packed_weights_torch(prob, "cuda").cpu().numpy()
        want = dg.packed_weights_np(prob)
        assert np.array_equal(_bits(got), _bits(want)), name
    prob = dg.make_problem("mixed", B=4, T=2, rows_cap=50_000)
    got = dg.packed_weights_torch(prob, "cuda").cpu().numpy()
    want = dg.packed_weights_np(prob)
    assert np.array_equal(_bits(got), _bits(want))
    sub = (np.abs(want.astype(np.float32)) < 2.0 ** -14) & (want != 0)
    assert sub.any()
