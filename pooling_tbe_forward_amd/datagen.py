"""Seeded synthetic inputs for the table-batched embedding-bag (TBE) operator.

This module is the one piece shared by the HIP path's callers and by the CPU
oracle's callers.  It only draws inputs (table shapes, bag lengths, ids,
per-sample weights, output gradients, embedding weights); it performs none of
the operator's arithmetic (no pooling, no sorting, no gradient math).

Input layout it produces follows the problem statement of the FBTriton TBE
article (ai.thesatyajit.com, "A lookup table that is most of the model"):

* one flat ``indices`` array holding every bag's ids;
* ``offsets`` with T*B+1 entries, laid out feature-major, so bag (t, b) is
  ``indices[offsets[t*B+b] : offsets[t*B+b+1]]``;
* every table packed row-major into one weight buffer, table after table.

Random streams: ``numpy.random.default_rng([seed, purpose, ...])`` with
purpose 0 = table shapes, 2 = bag lengths, 3 = ids (per table), 4 = per-sample
weights, 5 = output gradient.  Embedding weights (purpose 1) come from a
counter-based generator, ``lowbias32`` (Chris Wellons' integer hash), keyed on
(seed, table, element index), so that any row can be regenerated on the host
without materialising a multi-GB table, and a whole table is built on the GPU
with identical bits by one kernel launch (``gen/weights_gen.hip``, built into
``libtbe_datagen.so``; that library holds only this generator).  A weight value is an Irwin-Hall sum of four 16-bit
uniforms, centred and scaled to the configured standard deviation (an
approximately normal law), or a 24-bit uniform on [-1, 1).
"""
from __future__ import annotations

import dataclasses
import math
import os
from typing import Optional

import numpy as np

M32 = 0xFFFFFFFF

# --------------------------------------------------------------------------
# Workload recipes.  Shapes follow the five configurations this operator is
# measured and checked on; see the module docstring for the stream layout.
# --------------------------------------------------------------------------
CONFIGS = {
    # Three tables of different widths, a handful of bags, one forced empty bag
    # and one forced repeated id.
    "toy": dict(seed=100, T=3, B=4, rows=[100, 50, 20], dims=[8, 16, 4],
                wdtype="f32", wdist=("uniform", -1.0, 1.0),
                lengths=("uniform_int", 0, 5), ids="uniform",
                weighted="none", lr=0.1, force_toy=True),
    # Eight 1M-row D=128 fp32 tables, Poisson(20) bags, uniform ids.
    "uniform": dict(seed=101, T=8, B=2048, rows=[1_000_000] * 8, dims=[128] * 8,
                    wdtype="f32", wdist=("normal", 0.01),
                    lengths=("poisson", 20.0), ids="uniform",
                    weighted="none", lr=0.1),
    # Forty features, log-uniform rows, D in {64,128,256}, fp16, geometric bags,
    # Zipf(1.1) ids, per-sample weights on the first 20 features.
    "mixed": dict(seed=102, T=40, B=4096, rows=("loguniform", 1e4, 1e7),
                  dims=("choice", [64, 128, 256]), wdtype="f16",
                  wdist=("normal", 0.01), lengths=("geometric", 30.0, 500),
                  ids=("zipf", 1.1), weighted=("first", 20), lr=0.1),
    # One 64-row D=128 fp16 table, 16384 bags of exactly 256 ids.
    "hist": dict(seed=103, T=1, B=16384, rows=[64], dims=[128], wdtype="f16",
                 wdist=("normal", 0.1), lengths=("const", 256), ids="uniform",
                 weighted="none", lr=0.1),
    # Four 1M-row D=128 fp32 tables, 8192 bags of 50 Zipf(1.2) ids, weighted.
    "stress": dict(seed=104, T=4, B=8192, rows=[1_000_000] * 4, dims=[128] * 4,
                   wdtype="f32", wdist=("normal", 0.01), lengths=("const", 50),
                   ids=("zipf", 1.2), weighted="all", lr=0.1),
    # The stress shape with every touched row read a number of times uniform
    # in 32..255 (the band where the pages' threshold result sits).
    "band": dict(seed=105, T=4, B=8192, rows=[1_000_000] * 4, dims=[128] * 4,
                 wdtype="f32", wdist=("normal", 0.01), lengths=("const", 50),
                 ids=("band", 32, 255), weighted="all", lr=0.1),
    # Production-scale batch shaped like the statistics the pages quote (about
    # 4.2M bags, B = 128K, ~20 ids per bag, ~3M distinct rows, one row read
    # ~1e5 times): 32 features of 100K rows, D=128 fp16, Zipf(1.05) ids.
    "prod": dict(seed=106, T=32, B=131072, rows=[100_000] * 32, dims=[128] * 32,
                 wdtype="f16", wdist=("normal", 0.01), lengths=("poisson", 20.0),
                 ids=("zipf_cdf", 1.05), weighted="none", lr=0.1),
}


@dataclasses.dataclass
class Problem:
    """One seeded TBE problem instance (host arrays)."""
    name: str
    seed: int
    T: int
    B: int
    rows: np.ndarray          # int64 [T]
    dims: np.ndarray          # int32 [T]
    wdtype: str               # "f32" | "f16"
    wdist: tuple
    weighted: np.ndarray      # bool [T]
    lengths: np.ndarray       # int64 [T, B]
    offsets: np.ndarray       # int64 [T*B+1]
    indices: np.ndarray       # int64 [N]
    psw: Optional[np.ndarray]   # float32 [N] or None (unweighted problem)
    grad: np.ndarray          # float32 [B, sum(dims)]
    lr: float

    @property
    def N(self) -> int:
        return int(self.offsets[-1])

    @property
    def sum_D(self) -> int:
        return int(self.dims.sum())

    @property
    def np_wdtype(self):
        return np.float32 if self.wdtype == "f32" else np.float16

    def table_of_lookup(self) -> np.ndarray:
        """Feature id of every lookup (input bookkeeping, int64 [N])."""
        per_t = self.lengths.sum(axis=1)
        return np.repeat(np.arange(self.T, dtype=np.int64), per_t)

    def summary(self) -> dict:
        lens = self.lengths.ravel()
        return dict(name=self.name, seed=self.seed, T=self.T, B=self.B, N=self.N,
                    sum_rows=int(self.rows.sum()), sum_D=self.sum_D,
                    weight_bytes=int((self.rows * self.dims).sum()) *
                    (4 if self.wdtype == "f32" else 2),
                    max_bag=int(lens.max()) if lens.size else 0,
                    empty_bags=int((lens == 0).sum()),
                    weighted_tables=int(self.weighted.sum()))


# --------------------------------------------------------------------------
# Counter-based weight generator (host numpy and device torch, same bits).
# --------------------------------------------------------------------------
def _mul32(x, c):
    """(x * c) mod 2**32 for a Python int 0 <= x < 2**32."""
    return (x * c) & M32


def _lowbias32(x):
    """Chris Wellons' lowbias32 integer hash of a Python int in [0, 2**32)."""
    x ^= x >> 16
    x = _mul32(x, 0x7FEB352D)
    x ^= x >> 15
    x = _mul32(x, 0x846CA68B)
    x ^= x >> 16
    return x


def _lowbias32_u64(x):
    """lowbias32 of every element of a uint64 array of 32-bit values, in place
    (uint64 products are exact modulo 2**64, so masking keeps the low word)."""
    m = np.uint64(M32)
    x ^= x >> np.uint64(16)
    x *= np.uint64(0x7FEB352D)
    x &= m
    x ^= x >> np.uint64(15)
    x *= np.uint64(0x846CA68B)
    x &= m
    x ^= x >> np.uint64(16)
    return x


def _stream_key(seed: int, t: int, lane: int) -> int:
    k = (seed * 0x9E3779B9 + t * 0x85EBCA6B + lane * 0xC2B2AE35 + 0x27D4EB2F) & M32
    return int(_lowbias32(k))


def _ih_scale(sigma: float) -> float:
    # standard deviation of a sum of four independent uniforms on {0..65535}
    return sigma / math.sqrt(4.0 * (65536.0 ** 2 - 1.0) / 12.0)


def _dist_code(wdist):
    """(kind, scale) of a weight law: kind 0 = approximately normal with
    standard deviation wdist[1], kind 1 = uniform on [-1, 1)."""
    if wdist[0] == "normal":
        return 0, _ih_scale(float(wdist[1]))
    if wdist[0] == "uniform":
        assert (float(wdist[1]), float(wdist[2])) == (-1.0, 1.0), "only U(-1,1) is generated"
        return 1, 2.0 ** -24
    raise ValueError(wdist)


def _hash_elems_np(e, seed, t):
    """Two 32-bit hash words (uint64 arrays) per element index e >= 0."""
    e = np.asarray(e, dtype=np.int64).astype(np.uint64)
    e_lo = e & np.uint64(M32)
    e_hi = e >> np.uint64(32)
    out = []
    for lane in (0, 1):
        h = e_lo ^ np.uint64(_stream_key(seed, t, lane))
        h = _lowbias32_u64(h)
        h ^= e_hi
        out.append(_lowbias32_u64(h))
    return out


def _rows_block(seed, t, D, kind, scale, f16, r):
    e = (r[:, None] * D + np.arange(D, dtype=np.int64)[None, :]).reshape(-1)
    h0, h1 = _hash_elems_np(e, seed, t)
    if kind == 0:
        s = (h0 & np.uint64(0xFFFF)) + (h0 >> np.uint64(16)) + (h1 & np.uint64(0xFFFF)) + \
            (h1 >> np.uint64(16))
        v = (s.astype(np.int64) - 131070).astype(np.float64) * scale
    else:
        u24 = (h0 >> np.uint64(8)).astype(np.int64)
        v = (2 * u24 - (1 << 24)).astype(np.float64) * scale
    v = v.astype(np.float32)
    return v.astype(np.float16) if f16 else v


def weight_rows(prob: Problem, t: int, row_ids) -> np.ndarray:
    """Rows ``row_ids`` of table t as a [len, D_t] array of the weight dtype.

    Element e = row * D_t + column gets the hash words h0, h1 of
    _hash_elems_np; the value is computed in float64, rounded to float32 and,
    for fp16 tables, rounded once more to float16.  Work goes in blocks of
    about 64K elements, so the temporaries stay in cache."""
    D = int(prob.dims[t])
    r = np.asarray(row_ids, dtype=np.int64).reshape(-1)
    kind, scale = _dist_code(prob.wdist)
    f16 = prob.wdtype == "f16"
    out = np.empty((r.size, D), dtype=np.float16 if f16 else np.float32)
    step = max(1, 65536 // D)
    for s in range(0, r.size, step):
        e = min(s + step, r.size)
        out[s:e] = _rows_block(prob.seed, t, D, kind, scale, f16, r[s:e]).reshape(-1, D)
    return out


_gen_lib = None
GEN_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtbe_datagen.so")


def _gen():
    """libtbe_datagen.so: the device half of this generator (built with the
    package; see gen/weights_gen.hip)."""
    global _gen_lib
    if _gen_lib is None:
        import ctypes
        if not os.path.exists(GEN_LIB_PATH):
            raise RuntimeError(f"{GEN_LIB_PATH} is not built; run "
                               "`python -m pooling_tbe_forward_amd.build`")
        L = ctypes.CDLL(GEN_LIB_PATH)
        L.tbe_datagen_fill.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int32,
                                       ctypes.c_double, ctypes.c_void_p]
        L.tbe_datagen_fill.restype = ctypes.c_int
        _gen_lib = L
    return _gen_lib


def table_weights_torch(prob: Problem, t: int, out):
    """Fill the 1-D torch tensor ``out`` (rows_t*D_t elements) with table t:
    one kernel launch on a GPU tensor, the host generator otherwise."""
    import torch
    n = int(prob.rows[t]) * int(prob.dims[t])
    assert out.numel() == n and out.is_contiguous()
    if not out.is_cuda:
        out.copy_(torch.from_numpy(weight_rows(prob, t, np.arange(int(prob.rows[t]))).reshape(-1)))
        return out
    import ctypes
    kind, scale = _dist_code(prob.wdist)
    f16 = 1 if prob.wdtype == "f16" else 0
    assert out.dtype == (torch.float16 if f16 else torch.float32)
    rc = _gen().tbe_datagen_fill(ctypes.c_void_p(out.data_ptr()), n, f16,
                                 _stream_key(prob.seed, t, 0), _stream_key(prob.seed, t, 1),
                                 kind, scale,
                                 ctypes.c_void_p(torch.cuda.current_stream(out.device).cuda_stream))
    if rc != 0:
        raise RuntimeError(f"tbe_datagen_fill failed (hip error {rc})")
    return out


def table_element_starts(prob: Problem) -> np.ndarray:
    """Element offset of each table inside the packed input buffer (int64 [T+1]).

    This is the packing convention of the input format: table after table, each
    row-major with stride D_t.
    """
    sizes = prob.rows.astype(np.int64) * prob.dims.astype(np.int64)
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)


def packed_weights_torch(prob: Problem, device):
    """All tables packed into one 1-D torch tensor on ``device``."""
    import torch
    starts = table_element_starts(prob)
    dt = torch.float32 if prob.wdtype == "f32" else torch.float16
    w = torch.empty(int(starts[-1]), dtype=dt, device=device)
    for t in range(prob.T):
        table_weights_torch(prob, t, w[int(starts[t]):int(starts[t + 1])])
    return w


def packed_weights_np(prob: Problem) -> np.ndarray:
    """All tables packed into one host array (small problems only)."""
    parts = [weight_rows(prob, t, np.arange(int(prob.rows[t]))).reshape(-1)
             for t in range(prob.T)]
    return np.concatenate(parts) if parts else np.zeros(0, prob.np_wdtype)


# --------------------------------------------------------------------------
# Index / length / weight / gradient draws.
# --------------------------------------------------------------------------
def _zipf_bounded(rng, a: float, R: int, n: int) -> np.ndarray:
    """n draws of Zipf(a) restricted to ranks 1..R (rejection), minus one."""
    out = np.empty(n, dtype=np.int64)
    filled = 0
    while filled < n:
        need = n - filled
        d = rng.zipf(a, size=max(1024, int(need * 1.6) + 16))
        d = d[(d >= 1) & (d <= R)]
        take = min(need, d.size)
        out[filled:filled + take] = d[:take] - 1
        filled += take
    return out


def _zipf_cdf(rng, a: float, R: int, n: int) -> np.ndarray:
    """n draws of the Zipf(a) law bounded to ranks 1..R, by inverting its
    cumulative distribution (p_k proportional to k^-a), minus one: the same
    law as _zipf_bounded, drawn without rejection (for very large n)."""
    cdf = np.cumsum(np.arange(1, R + 1, dtype=np.float64) ** -a)
    u = rng.random(n) * cdf[-1]
    return np.minimum(np.searchsorted(cdf, u, side="right"), R - 1).astype(np.int64)


def _band_ids(rng, lo: int, hi: int, R: int, n: int) -> np.ndarray:
    """n ids in which every id used is read a number of times drawn uniformly
    from lo..hi (the last one is cut to fill exactly n), in random order."""
    counts = []
    total = 0
    while total < n:
        c = int(rng.integers(lo, hi + 1))
        c = min(c, n - total)
        counts.append(c)
        total += c
    rows = rng.choice(R, size=len(counts), replace=False).astype(np.int64)
    return rng.permutation(np.repeat(rows, counts))


def _rng(seed: int, batch: int, *key):
    """Stream for one purpose; batch 0 keeps the base streams, other batches
    draw fresh lengths / ids / weights / gradients over the same tables."""
    if batch == 0:
        return np.random.default_rng([seed, *key])
    return np.random.default_rng([seed, *key, 1000 + int(batch)])


def make_problem(name: str, seed: Optional[int] = None, B: Optional[int] = None,
                 rows_cap: Optional[int] = None, T: Optional[int] = None,
                 weighted: Optional[str] = None, wdtype: Optional[str] = None,
                 batch: int = 0) -> Problem:
    """Build a seeded problem from a named recipe; optional size overrides
    (``B``, ``T``, ``rows_cap``) give smaller instances of the same shape, and
    ``batch`` selects another batch of lookups over the same tables."""
    cfg = dict(CONFIGS[name])
    seed = cfg["seed"] if seed is None else int(seed)
    Tn = cfg["T"] if T is None else int(T)
    Bn = cfg["B"] if B is None else int(B)

    rng0 = np.random.default_rng([seed, 0])
    rspec = cfg["rows"]
    if isinstance(rspec, tuple) and rspec[0] == "loguniform":
        rows = np.floor(np.exp(rng0.uniform(math.log(rspec[1]), math.log(rspec[2]),
                                            size=cfg["T"]))).astype(np.int64)
    else:
        rows = np.asarray(rspec, dtype=np.int64)
    dspec = cfg["dims"]
    if isinstance(dspec, tuple) and dspec[0] == "choice":
        dims = rng0.choice(np.asarray(dspec[1]), size=cfg["T"]).astype(np.int32)
    else:
        dims = np.asarray(dspec, dtype=np.int32)
    rows = rows[:Tn].copy()
    dims = dims[:Tn].copy()
    if rows_cap is not None:
        rows = np.minimum(rows, int(rows_cap))

    rng2 = _rng(seed, batch, 2)
    lspec = cfg["lengths"]
    if lspec[0] == "uniform_int":
        lengths = rng2.integers(lspec[1], lspec[2] + 1, size=(Tn, Bn))
    elif lspec[0] == "poisson":
        lengths = rng2.poisson(lspec[1], size=(Tn, Bn))
    elif lspec[0] == "geometric":
        lengths = np.minimum(rng2.geometric(1.0 / lspec[1], size=(Tn, Bn)), lspec[2])
    elif lspec[0] == "const":
        lengths = np.full((Tn, Bn), lspec[1])
    else:
        raise ValueError(lspec)
    lengths = lengths.astype(np.int64)
    if cfg.get("force_toy"):
        # bag (t=1, b=2) empty; bag (0, 0) holds at least two ids, second = first
        if Tn > 1 and Bn > 2:
            lengths[1, 2] = 0
        lengths[0, 0] = max(int(lengths[0, 0]), 2)

    ids = []
    for t in range(Tn):
        n_t = int(lengths[t].sum())
        rng3 = _rng(seed, batch, 3, t)
        R = int(rows[t])
        if cfg["ids"] == "uniform":
            it = rng3.integers(0, R, size=n_t, dtype=np.int64)
        elif isinstance(cfg["ids"], tuple) and cfg["ids"][0] == "zipf":
            it = _zipf_bounded(rng3, float(cfg["ids"][1]), R, n_t)
        elif isinstance(cfg["ids"], tuple) and cfg["ids"][0] == "zipf_cdf":
            it = _zipf_cdf(rng3, float(cfg["ids"][1]), R, n_t)
        elif isinstance(cfg["ids"], tuple) and cfg["ids"][0] == "band":
            it = _band_ids(rng3, int(cfg["ids"][1]), int(cfg["ids"][2]), R, n_t)
        else:
            raise ValueError(cfg["ids"])
        if cfg.get("force_toy") and t == 0 and n_t >= 2:
            it[1] = it[0]
        ids.append(it)
    indices = np.concatenate(ids) if ids else np.zeros(0, np.int64)
    offsets = np.concatenate([[0], np.cumsum(lengths.ravel())]).astype(np.int64)

    wspec = cfg["weighted"] if weighted is None else weighted
    if wspec == "none":
        wmask = np.zeros(Tn, dtype=bool)
    elif wspec == "all":
        wmask = np.ones(Tn, dtype=bool)
    elif isinstance(wspec, tuple) and wspec[0] == "first":
        wmask = np.arange(Tn) < wspec[1]
    else:
        raise ValueError(wspec)
    N = int(offsets[-1])
    psw = None
    if wmask.any():
        psw = _rng(seed, batch, 4).random(N, dtype=np.float32)
        # lookups of unweighted features carry weight exactly 1
        tl = np.repeat(np.arange(Tn), lengths.sum(axis=1))
        psw[~wmask[tl]] = np.float32(1.0)

    grad = _rng(seed, batch, 5).standard_normal(
        (Bn, int(dims.sum())), dtype=np.float32)

    return Problem(name=name, seed=seed, T=Tn, B=Bn, rows=rows, dims=dims,
                   wdtype=cfg["wdtype"] if wdtype is None else wdtype,
                   wdist=cfg["wdist"], weighted=wmask,
                   lengths=lengths, offsets=offsets, indices=indices, psw=psw,
                   grad=grad, lr=float(cfg["lr"]))


def sample_prefix(prob: Problem, Bs: int) -> Problem:
    """The same batch restricted to samples 0..Bs-1 of every feature (a
    bounded sample of a workload): bag (t, b) of the result is bag (t, b) of
    ``prob`` for b < Bs, with its ids, per-sample weights and output-gradient
    row.  Input bookkeeping only."""
    Bs = min(int(Bs), prob.B)
    lengths = prob.lengths[:, :Bs].copy()
    parts_i, parts_w = [], []
    for t in range(prob.T):
        s, e = int(prob.offsets[t * prob.B]), int(prob.offsets[t * prob.B + Bs])
        parts_i.append(prob.indices[s:e])
        if prob.psw is not None:
            parts_w.append(prob.psw[s:e])
    offsets = np.concatenate([[0], np.cumsum(lengths.ravel())]).astype(np.int64)
    return dataclasses.replace(
        prob, B=Bs, lengths=lengths, offsets=offsets,
        indices=np.concatenate(parts_i) if parts_i else np.zeros(0, np.int64),
        psw=np.concatenate(parts_w) if prob.psw is not None else None,
        grad=np.ascontiguousarray(prob.grad[:Bs]))


def exact_problem(seed: int, T: int = 3, B: int = 37, max_rows: int = 40,
                  dims=(8, 16, 4), wdtype: str = "f32", weighted: bool = True,
                  max_len: int = 9):
    """A small problem whose every partial sum is exactly representable.

    Weights are integers in [-8, 8], per-sample weights are in
    {0.25, 0.5, 1, 2}, output gradients are integers in [-4, 4], and the
    learning rate is 0.5, so any summation order yields the same bits.
    Returns (problem, packed host weights).
    """
    rng = np.random.default_rng([seed, 77])
    dims = np.asarray(list(dims)[:T], dtype=np.int32)
    rows = rng.integers(1, max_rows + 1, size=T).astype(np.int64)
    lengths = rng.integers(0, max_len + 1, size=(T, B)).astype(np.int64)
    ids = [rng.integers(0, rows[t], size=int(lengths[t].sum()), dtype=np.int64)
           for t in range(T)]
    indices = np.concatenate(ids)
    offsets = np.concatenate([[0], np.cumsum(lengths.ravel())]).astype(np.int64)
    N = int(offsets[-1])
    wmask = np.ones(T, dtype=bool) if weighted else np.zeros(T, dtype=bool)
    psw = (rng.choice(np.asarray([0.25, 0.5, 1.0, 2.0], np.float32), size=N)
           if weighted else None)
    grad = rng.integers(-4, 5, size=(B, int(dims.sum()))).astype(np.float32)
    npdt = np.float32 if wdtype == "f32" else np.float16
    packed = rng.integers(-8, 9, size=int((rows * dims).sum())).astype(npdt)
    prob = Problem(name="exact", seed=seed, T=T, B=B, rows=rows, dims=dims,
                   wdtype=wdtype, wdist=("explicit",), weighted=wmask,
                   lengths=lengths, offsets=offsets, indices=indices, psw=psw,
                   grad=grad, lr=0.5)
    return prob, packed
