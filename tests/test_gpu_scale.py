"""Production-scale check: one batch shaped like the statistics the pages
quote for a production shard (83.9M lookups over 32 features, B = 131,072,
3.0M distinct rows, 28 lookups per distinct row on average, hottest row read
282K times), run through the C ABI in the launch configuration the benchmark
times:

* forward: every element of the [131072, 4096] output against the oracle;
* integer stage: sorted keys and positions, unique keys, run starts and
  lengths, short / long lists bit-exact against the oracle, all 83.9M keys;
* backward-SGD: every updated row within tolerance of the oracle, every
  other row bit-identical to the generator.
"""
import numpy as np
import pytest
import torch

from pooling_tbe_forward_amd import datagen as dg
from tests import fullcheck
from tests import helpers as H
from tests.test_gpu_backward import _compare_sort, gpu_backward, gpu_sort
from tests.test_gpu_forward import _run_forward

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def test_production_scale_forward_sort_backward():
    prob = dg.make_problem("prod")
    print(f"prod: N={prob.N} T={prob.T} B={prob.B}", flush=True)
    w_dev = dg.packed_weights_torch(prob, "cuda")
    out = _run_forward(prob, w_dev)
    assert np.isfinite(out).all()
    rep = fullcheck.forward_all(prob, out)
    assert rep["ok"], rep
    del out

    o = H.oracle_sort(prob, 64)
    _compare_sort(gpu_sort(prob, tau=64), o, prob.N)
    del o

    gpu_backward(prob, w_dev)
    rep = fullcheck.backward_all(prob, w_dev)
    assert rep["ok"], rep
    fullcheck.untouched_all(prob, w_dev)
    del w_dev
    torch.cuda.empty_cache()
