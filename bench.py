#!/usr/bin/env python
"""Benchmark of the TBE hot path on one MI355X.

One step = forward pooled sum + backward with exact SGD over one batch of the
mixed production-like workload (40 features, rows log-uniform in 1e4..1e7,
D in {64, 128, 256} fp16, B = 4096, geometric(30) bags capped at 500,
Zipf(1.1) ids, per-sample weights on 20 features; 4.93M lookups per batch),
the largest configuration this operator is measured on.  Prints ONE JSON line
on stdout; the uniform workload (8 x 1M-row D=128 fp32 tables, B = 2048,
Poisson(20) bags) is measured the same way and nested in it.

* Inputs are resident in HBM before the timed region.  Consecutive steps cycle
  through several distinct batches over the same tables ("warm": what a
  training loop sees; the Zipf-hot rows of one batch are hot in the next).
  A "cold" run puts an untimed read of 1 GiB (four times the 256 MB
  on-package cache) before each forward and before each backward, so every
  pass starts with nothing of the previous one in any cache.
* The step's schedule (--schedule): by default each step (forward, then
  backward-SGD) is launched eagerly on one stream ("eager"); "graph" captures
  each batch's step once in a HIP graph and replays it; "serial" is the eager
  schedule with the library's stage events recorded (they add a few
  microseconds per event); "overlap" runs the backward's integer stage (key
  pass, radix sort, run-length encode; it reads only the batch's indices) on a
  second stream while the forward runs.  All four are timed; the JSON line
  carries every step time, and the per-stage times come from the "serial" run.
* Stage times come from HIP events that the library records on its streams at
  its own stage boundaries (tbe_set_stage_events), so the dominant kernel's
  duration is measured live inside the timed region.
* The JSON line also carries "adagrad": the same steps with exact row-wise
  Adagrad in the backward (tbe_backward_adagrad, one fp32 state per row);
  "mean_pooling": the SGD steps on a mean-pooled plan; "int64_indices": the
  SGD steps with int64 indices and offsets; and "cpu_baseline": the CPU oracle
  on a bounded sample of the same workload, on one host thread and on all of
  the process's host threads (OpenMP).
* --report also prints one JSON line per configuration (uniform, mixed, hist,
  stress, band, prod) with forward / backward stage times on stderr;
  --tau / --chunk set the long-run threshold and chunk for a sweep.
* --calibrate-copy runs a 1 GiB device copy (for scaling rocprofv3 byte
  counters); --summarize-pmc turns rocprofv3 --pmc CSVs into the traffic
  summary under profiles/ that the roofline's "traffic" field reads.
"""
from __future__ import annotations

import argparse
import ctypes
import csv
import glob
import hashlib
import json
import os
import platform
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PEAK_MFMA_F16_TFLOPS = 2500.0   # dense fp16 matrix peak of an MI355X
SEGMENT_SRC = os.path.join(ROOT, "pooling_tbe_forward_amd", "csrc", "bwd_segment.hip")
FLUSH_BYTES = 1 << 30           # the cold runs' cache flush: larger than the 256 MB MALL


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"traffic_k_segment_{workload}.json")


WORKLOAD_DESC = {
    "uniform": "uniform TBE: T=8 tables x 1,000,000 rows, D=128 fp32, B=2048, "
               "Poisson(20) bags, uniform ids, unweighted, forward + backward exact SGD",
    "mixed": "mixed production-like TBE: T=40 features, rows log-uniform 1e4..1e7, "
             "D in {64,128,256} fp16, B=4096, geometric(30) bags capped at 500, Zipf(1.1) ids, "
             "per-sample weights on 20 features, forward + backward exact SGD",
    "hist": "small-table TBE: T=1 x 64 rows, D=128 fp16, B=16384, 256 ids per bag",
    "stress": "run-length stress TBE: T=4 x 1,000,000 rows, D=128 fp32, B=8192, 50 Zipf(1.2) "
              "ids per bag, weighted",
    "band": "band-planted TBE: the run-length stress shape with every touched row read "
            "32..255 times (uniform), weighted",
    "prod": "production-scale TBE: T=32 x 100,000 rows, D=128 fp16, B=131,072, Poisson(20) "
            "bags (83.9M lookups, 3.0M distinct rows), Zipf(1.05) ids, unweighted",
    "toy": "toy TBE: T=3, rows {100,50,20}, D {8,16,4}, B=4",
}
BWD_STAGES = ["keys", "radix_sort", "rle", "segment_sgd", "long_combine"]
SCHEDULE_DESC = {
    "eager": "tbe_forward then tbe_backward_sgd on one stream, launched eagerly",
    "graph": "tbe_forward then tbe_backward_sgd, captured once per batch in a HIP graph and "
             "replayed",
    "overlap": "backward integer stage (tbe_backward_prepare) on a second stream concurrently "
               "with tbe_forward, then tbe_backward_apply",
    "serial": "tbe_forward then tbe_backward_sgd on one stream, launched eagerly, with the "
              "library's stage events recorded (per-stage times)",
}


def radix_passes(sum_rows):
    """Radix passes the library's sort makes over keys of ceil(log2 sum_rows)
    bits (digits of at most 8 bits)."""
    bits = max(1, int(np.ceil(np.log2(max(2, int(sum_rows))))))
    return (bits + 7) // 8


def algorithmic_bytes(prob):
    """Bytes the method must move (int32 indices), per launch / per pass."""
    s_i = 4
    s_w = 4 if prob.wdtype == "f32" else 2
    TB = prob.T * prob.B
    tl = prob.table_of_lookup()
    N = prob.N
    n_w = int(prob.weighted[tl].sum()) if prob.psw is not None else 0
    hcs = np.concatenate([[0], np.cumsum(prob.rows)])
    keys = hcs[tl] + prob.indices
    uk = np.unique(keys)
    ut = np.searchsorted(hcs, uk, side="right") - 1
    uniq_row_bytes = int((prob.dims[ut].astype(np.int64) * s_w).sum())
    lookup_row_bytes = int((prob.dims[tl].astype(np.int64) * s_w).sum())
    out_bytes = prob.B * prob.sum_D * 4
    jag = N * s_i + (TB + 1) * s_i + n_w * 4
    passes = radix_passes(prob.rows.sum())
    payload = 8 if prob.psw is not None else 4
    sort_bytes = passes * N * (4 + payload) * 2
    run_bytes = uk.size * 16
    # segment-reduce + SGD kernel: every touched row read and written once,
    # grad_output read once, the sorted payload and the run records read once
    seg = 2 * uniq_row_bytes + out_bytes + N * payload + run_bytes
    # row-wise Adagrad adds one fp32 state read + write per touched row
    return dict(N=N, unique_rows=int(uk.size), passes=passes, seg_min_adagrad=seg + 8 * uk.size,
                fwd_min=jag + uniq_row_bytes + out_bytes,
                fwd_lookup=jag + lookup_row_bytes + out_bytes,
                bwd_min=jag + out_bytes + 2 * uniq_row_bytes + sort_bytes + run_bytes,
                seg_min=seg)


class Hip:
    """The HIP runtime torch loaded (events for the library's stage hook)."""

    def __init__(self):
        import torch
        path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
        if not os.path.exists(path):
            path = "libamdhip64.so"
        h = ctypes.CDLL(path)
        h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                          ctypes.c_void_p]
        h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.h = h

    def event(self):
        e = ctypes.c_void_p()
        assert self.h.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def record(self, ev, stream):
        assert self.h.hipEventRecord(ev, ctypes.c_void_p(stream.cuda_stream)) == 0

    def ms(self, a, b):
        v = ctypes.c_float()
        assert self.h.hipEventElapsedTime(ctypes.byref(v), a, b) == 0
        return float(v.value)

    def destroy(self, evs):
        for e in evs:
            self.h.hipEventDestroy(e)


class Workload:
    """Device-resident inputs for several batches over one set of tables.

    probs: the batches' host problems (made here when None); tuning: launch
    knobs for the plan (e.g. tau, chunk)."""

    def __init__(self, name, nbatches, index_dtype="i32", probs=None, tuning=None):
        import torch
        from pooling_tbe_forward_amd import datagen as dg
        from pooling_tbe_forward_amd import tbe
        self.name = name
        self.probs = probs or [dg.make_problem(name, batch=k) for k in range(nbatches)]
        p0 = self.probs[0]
        self.weights = dg.packed_weights_torch(p0, "cuda")
        self.plan = tbe.tbe_plan_create(p0.rows, p0.dims,
                                        tbe.TBE_F32 if p0.wdtype == "f32" else tbe.TBE_F16,
                                        tbe.TBE_I32 if index_dtype == "i32" else tbe.TBE_I64,
                                        weighted=p0.weighted)
        if tuning:
            tbe.tbe_set_tuning(self.plan, **tuning)
        it = torch.int32 if index_dtype == "i32" else torch.int64
        self.inputs = []
        for p in self.probs:
            self.inputs.append(dict(
                indices=torch.from_numpy(p.indices).to("cuda", it),
                offsets=torch.from_numpy(p.offsets).to("cuda", it),
                psw=None if p.psw is None else torch.from_numpy(p.psw).to("cuda"),
                grad=torch.from_numpy(p.grad).to("cuda")))
        ws = max(tbe.tbe_backward_workspace_bytes(self.plan, p.B, p.N) for p in self.probs)
        self.ws = tbe.tbe_workspace_init(torch.empty(ws, dtype=torch.uint8, device="cuda"))
        self.out = torch.empty(p0.B, p0.sum_D, dtype=torch.float32, device="cuda")
        # row-wise Adagrad state: one fp32 value per row of every table
        self.state = torch.zeros(int(np.sum(p0.rows)), dtype=torch.float32, device="cuda")
        self.bytes = [algorithmic_bytes(p) for p in self.probs]
        self.side = torch.cuda.Stream()          # default priority
        self.ev_start = torch.cuda.Event()
        self.ev_ready = torch.cuda.Event()
        self._flush = None
        torch.cuda.synchronize()

    def flush(self):
        """An untimed read of 1 GiB on the current stream: whatever the
        previous pass left in the L2s and the 256 MB MALL is evicted (dirty
        lines are written back during the flush, and it leaves none of its
        own for the next pass to write back)."""
        import torch
        if self._flush is None:
            self._flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        self._flush.sum()

    def close(self):
        self._flush = None

    def fwd(self, k, events=None):
        from pooling_tbe_forward_amd import tbe
        p, d = self.probs[k], self.inputs[k]
        if events:
            tbe.tbe_set_stage_events(self.plan, events)
        tbe.tbe_forward(self.plan, p.B, self.weights, d["indices"], d["offsets"], d["psw"],
                        self.out)

    def bwd(self, k, events=None):
        from pooling_tbe_forward_amd import tbe
        p, d = self.probs[k], self.inputs[k]
        if events:
            tbe.tbe_set_stage_events(self.plan, events)
        tbe.tbe_backward_sgd(self.plan, p.B, self.weights, d["indices"], d["offsets"], d["psw"],
                             d["grad"], p.lr, self.ws)

    def bwd_adagrad(self, k, events=None):
        from pooling_tbe_forward_amd import tbe
        p, d = self.probs[k], self.inputs[k]
        if events:
            tbe.tbe_set_stage_events(self.plan, events)
        tbe.tbe_backward_adagrad(self.plan, p.B, self.weights, self.state, d["indices"],
                                 d["offsets"], d["psw"], d["grad"], p.lr, self.ws)

    def step_overlapped(self, k, hip=None, fe=None, be=None):
        """The backward's integer stage on a second stream while the forward
        runs; the segment reduce + SGD follows both.  be[6] (if given) is
        recorded on the main stream right before the apply half starts."""
        import torch
        from pooling_tbe_forward_amd import tbe
        p, d = self.probs[k], self.inputs[k]
        main = torch.cuda.current_stream()
        self.ev_start.record(main)
        self.side.wait_event(self.ev_start)
        if be:
            tbe.tbe_set_stage_events(self.plan, be[:4])
        tbe.tbe_backward_prepare(self.plan, p.B, d["indices"], d["offsets"], d["psw"], self.ws,
                                 stream=self.side)
        if fe:
            tbe.tbe_set_stage_events(self.plan, fe)
        tbe.tbe_forward(self.plan, p.B, self.weights, d["indices"], d["offsets"], d["psw"],
                        self.out, stream=main)
        self.ev_ready.record(self.side)
        main.wait_event(self.ev_ready)
        if be:
            hip.record(be[6], main)
            tbe.tbe_set_stage_events(self.plan, [None] * 4 + be[4:6])
        tbe.tbe_backward_apply(self.plan, p.B, p.N, d["psw"] is not None, self.weights,
                               d["grad"], p.lr, self.ws, stream=main)


def run_steps(wl, steps, warmup, hip, overlap=False, adagrad=False, cold=False):
    """Warm up, then time `steps` steps (synchronize on both sides); per-stage
    HIP events recorded by the library on the streams it runs on.

    overlap=False: forward, then the whole backward, on one stream.
    overlap=True: the backward's integer stage (key pass, radix sort, RLE) on a
    second stream concurrently with the forward, then segment reduce + SGD.
    cold=True: an untimed cache flush before each forward and each backward
    (outside the stage events; the wall time then includes the flushes)."""
    import torch
    nb = len(wl.probs)
    bwd = wl.bwd_adagrad if adagrad else wl.bwd
    fl = wl.flush if cold else (lambda: None)

    def one(k, fe=None, be=None):
        if overlap:
            wl.step_overlapped(k, hip, fe, be)
            return
        fl()
        wl.fwd(k, fe)
        fl()
        bwd(k, be)

    for s in range(warmup):
        one(s % nb)
    torch.cuda.synchronize()
    fe = [[hip.event() for _ in range(2)] for _ in range(steps)]
    be = [[hip.event() for _ in range(7)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        one(s % nb, fe[s], be[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    f_ms = np.array([hip.ms(fe[s][0], fe[s][1]) for s in range(steps)])
    b_ms = np.array([hip.ms(be[s][0], be[s][5]) for s in range(steps)])
    stage_ms = np.array([[hip.ms(be[s][i], be[s][i + 1]) for i in range(5)]
                         for s in range(steps)])
    if overlap:   # the segment stage starts at the apply half, on the main stream
        stage_ms[:, 3] = [hip.ms(be[s][6], be[s][4]) for s in range(steps)]
    for s in range(steps):
        hip.destroy(fe[s] + be[s])
    ks = [s % nb for s in range(steps)]
    pick = lambda key: np.array([wl.bytes[k][key] for k in ks], dtype=np.float64)
    return dict(wall_s=wall, fwd_ms=f_ms, bwd_ms=b_ms, stage_ms=stage_ms, lookups=pick("N"),
                fwd_bytes=pick("fwd_min"), bwd_bytes=pick("bwd_min"),
                seg_bytes=pick("seg_min_adagrad" if adagrad else "seg_min"))


def run_plain_steps(wl, steps, warmup, adagrad=False):
    """Forward then backward (exact SGD, or row-wise Adagrad) per step on the
    current stream, no timing events: warm-up, then `steps` timed steps
    between two synchronizations."""
    import torch
    nb = len(wl.probs)
    bwd = wl.bwd_adagrad if adagrad else wl.bwd
    for s in range(warmup):
        wl.fwd(s % nb)
        bwd(s % nb)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        wl.fwd(s % nb)
        bwd(s % nb)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ks = [s % nb for s in range(steps)]
    return dict(wall_s=wall, lookups=np.array([wl.bytes[k]["N"] for k in ks], dtype=np.float64))


def stage_us(r):
    return {k: round(1e3 * float(v), 2) for k, v in zip(BWD_STAGES, r["stage_ms"].mean(axis=0))}


def adagrad_summary(wl, steps, warmup, hip):
    """The same steps with row-wise Adagrad in the backward: plain eager step
    time, and the backward's stage times and segment-kernel rate from a run
    with stage events."""
    r = run_steps(wl, steps, warmup, hip, adagrad=True)
    rp = run_plain_steps(wl, steps, warmup, adagrad=True)
    seg_us = float(np.mean(r["stage_ms"][:, 3])) * 1e3
    seg_gbps = float(np.mean(r["seg_bytes"])) / (seg_us * 1e-6) / 1e9
    return dict(step_ms_eager=1e3 * rp["wall_s"] / steps,
                lookups_per_s=float(np.sum(rp["lookups"])) / rp["wall_s"],
                bwd_ms=float(np.mean(r["bwd_ms"])), bwd_stage_us=stage_us(r),
                segment_gbps_min=round(seg_gbps, 1),
                segment_pct_peak=round(100 * seg_gbps / PEAK_HBM_GBPS, 2))


def mean_pooling_summary(wl, steps, warmup, hip):
    """The same SGD steps on a mean-pooled plan (tbe_plan_set_pooling): plain
    eager step time and the stage times of a run with stage events."""
    from pooling_tbe_forward_amd import tbe
    tbe.tbe_plan_set_pooling(wl.plan, "mean")
    try:
        r = run_steps(wl, steps, warmup, hip)
        rp = run_plain_steps(wl, steps, warmup)
    finally:
        tbe.tbe_plan_set_pooling(wl.plan, "sum")
    return dict(step_ms_eager=1e3 * rp["wall_s"] / steps,
                lookups_per_s=float(np.sum(rp["lookups"])) / rp["wall_s"],
                fwd_ms=float(np.mean(r["fwd_ms"])), bwd_ms=float(np.mean(r["bwd_ms"])),
                bwd_stage_us=stage_us(r))


def int64_summary(config, probs, steps, warmup, hip):
    """The same batches with int64 indices and offsets (a plan of index type
    TBE_I64, its own copy of the tables): plain eager step time and the stage
    times of a run with stage events."""
    import torch
    wl = Workload(config, len(probs), index_dtype="i64", probs=probs)
    r = run_steps(wl, steps, warmup, hip)
    rp = run_plain_steps(wl, steps, warmup)
    res = dict(step_ms_eager=1e3 * rp["wall_s"] / steps,
               lookups_per_s=float(np.sum(rp["lookups"])) / rp["wall_s"],
               fwd_ms=float(np.mean(r["fwd_ms"])), bwd_ms=float(np.mean(r["bwd_ms"])),
               bwd_stage_us=stage_us(r))
    del wl
    torch.cuda.empty_cache()
    return res


def capture_steps(wl):
    """One HIP graph per batch, each holding that batch's whole step (forward,
    then backward-SGD: the library's kernels only, no host work)."""
    import torch
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()          # default priority
    graphs = []
    for k in range(len(wl.probs)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            wl.fwd(k)
            wl.bwd(k)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def run_graph_steps(wl, graphs, steps, warmup):
    """Replay the captured steps: warm-up, then `steps` timed replays between
    two synchronizations."""
    import torch
    nb = len(graphs)
    for s in range(warmup):
        graphs[s % nb].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        graphs[s % nb].replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ks = [s % nb for s in range(steps)]
    return dict(wall_s=wall, lookups=np.array([wl.bytes[k]["N"] for k in ks], dtype=np.float64))


def host_cpu():
    cpu = platform.processor() or platform.machine()
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return cpu


def host_threads():
    """Threads this process may use: its CPU affinity, at most 16 (the host
    share of one GPU on the machines this runs on)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(config="mixed", budget_s=20.0, samples=256):
    """The CPU oracle, as it stands, on a bounded sample of the workload:
    samples 0..samples-1 of every feature of batch 0 (forward of those bags,
    the integer stage over their lookups, backward-SGD of every row they
    touch; the touched rows are regenerated on the host, untimed).  Timed on
    one host thread and again with the oracle's OpenMP loops on every thread
    the process may use, each leg repeated within about half the budget."""
    import oracle
    from pooling_tbe_forward_amd import datagen as dg
    full = dg.make_problem(config)
    prob = dg.sample_prefix(full, samples)
    tl = prob.table_of_lookup()
    rowsets = [np.unique(prob.indices[tl == t]) for t in range(prob.T)]
    tabs = [(ids, np.ascontiguousarray(dg.weight_rows(prob, t, ids).reshape(-1)))
            for t, ids in enumerate(rowsets)]
    code = oracle.F32 if prob.wdtype == "f32" else oracle.F16

    def leg(threads, budget):
        oracle.set_threads(threads)
        reps, total = 0, 0.0
        stage = dict(forward=0.0, sort_rle=0.0, backward=0.0)
        while total < budget and reps < 50:
            t0 = time.perf_counter()
            oracle.forward(prob.T, prob.B, prob.rows, prob.dims, code, tabs, prob.indices,
                           prob.offsets, prob.psw, prob.weighted)
            t1 = time.perf_counter()
            r = oracle.sort_rle(prob.T, prob.B, prob.rows, prob.indices, prob.offsets, 64)
            t2 = time.perf_counter()
            oracle.backward_sgd(prob.T, prob.B, prob.rows, prob.dims, code, tabs, prob.indices,
                                prob.offsets, prob.psw, prob.weighted, prob.grad, prob.lr,
                                r["unique_keys"])
            t3 = time.perf_counter()
            stage["forward"] += t1 - t0
            stage["sort_rle"] += t2 - t1
            stage["backward"] += t3 - t2
            total += t3 - t0
            reps += 1
        return dict(value=prob.N * reps / total, cores=threads, reps=reps,
                    ms_per_step=1e3 * total / reps,
                    stage_ms={k: round(1e3 * v / reps, 3) for k, v in stage.items()})

    nthr = host_threads()
    try:
        one = leg(1, budget_s / 2)
        many = leg(nthr, budget_s / 2) if nthr > 1 else one
    finally:
        oracle.set_threads(1)
    return dict(value=many["value"], unit="lookups/s", cores=many["cores"], kind="oracle",
                sample=f"{config} batch 0, samples 0..{prob.B - 1} of all {prob.T} features "
                       f"({prob.T * prob.B} bags, {prob.N} lookups, {sum(r.size for r in rowsets)} "
                       f"distinct rows): forward of every bag, sort+RLE of every lookup, "
                       f"backward-SGD of every touched row; fp64 accumulation; value = the "
                       f"OpenMP leg",
                ms_per_step=many["ms_per_step"], stage_ms=many["stage_ms"], reps=many["reps"],
                single_thread=one, host_cpu=host_cpu(), host_threads=nthr,
                nproc=os.cpu_count())


def source_hash(path):
    """sha256 prefix of a source file's code: comments and blank lines are
    dropped first, so an edit of the comments keeps counters taken on the
    same code valid."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


TRAFFIC_TUNING = ("tau", "chunk", "seg_slab_kib")


def plan_tuning(plan):
    from pooling_tbe_forward_amd import tbe
    t = tbe.tbe_get_tuning(plan)
    return {k: int(getattr(t, k)) for k in TRAFFIC_TUNING}


def measured_traffic(workload, tuning):
    """HBM bytes per k_segment launch from the committed PMC summary of this
    workload, or None when the kernel source or the launch knobs that shape
    its work (tuning: plan_tuning of the plan timed) changed since the
    counters were taken, or there is no summary."""
    try:
        t = json.load(open(traffic_file(workload)))
    except (OSError, ValueError):
        return None
    if t.get("source_sha256_16") != source_hash(SEGMENT_SRC):
        return None
    if t.get("tuning") != tuning:
        return None
    return t.get("traffic_bytes")


def summarize(r):
    f = float(np.mean(r["fwd_ms"]))
    b = float(np.mean(r["bwd_ms"]))
    lk = float(np.mean(r["lookups"]))
    out = dict(fwd_ms=f, bwd_ms=b, fwd_lookups_per_s=lk / (f * 1e-3),
               bwd_lookups_per_s=lk / (b * 1e-3),
               fwd_hbm_gbps_min=float(np.mean(r["fwd_bytes"])) / (f * 1e-3) / 1e9,
               bwd_hbm_gbps_min=float(np.mean(r["bwd_bytes"])) / (b * 1e-3) / 1e9,
               bwd_stage_us=stage_us(r))
    out["fwd_pct_peak"] = 100 * out["fwd_hbm_gbps_min"] / PEAK_HBM_GBPS
    out["bwd_pct_peak"] = 100 * out["bwd_hbm_gbps_min"] / PEAK_HBM_GBPS
    return out


def segment_roofline(r, workload, tuning):
    """Roofline entry of the dominant kernel, k_segment: its algorithmic bytes
    per launch over its average launch time from the library's stage events."""
    seg_us = float(np.mean(r["stage_ms"][:, 3])) * 1e3
    seg_bytes = float(np.mean(r["seg_bytes"]))
    seg_gbps = seg_bytes / (seg_us * 1e-6) / 1e9
    return dict(bound="hbm", kernel="k_segment (backward segment-reduce + SGD)",
                achieved=round(seg_gbps, 1), peak=PEAK_HBM_GBPS, unit="GB/s",
                frac=round(seg_gbps / PEAK_HBM_GBPS, 4), traffic=measured_traffic(workload, tuning),
                avg_launch_us=round(seg_us, 2), bytes_per_launch=int(seg_bytes))


def measure(wl, steps, warmup, hip, schedule, extras=True):
    """Every schedule of one workload, plus the cold run; returns the fields
    of its JSON object."""
    r_serial = run_steps(wl, steps, warmup, hip)
    r_over = run_steps(wl, steps, warmup, hip, overlap=True)
    r_graph = run_graph_steps(wl, capture_steps(wl), steps, warmup)
    r_eager = run_plain_steps(wl, steps, warmup)
    r_cold = run_steps(wl, max(5, steps // 2), 2, hip, cold=True)
    tun = plan_tuning(wl.plan)
    wl.close()
    r = dict(serial=r_serial, overlap=r_over, graph=r_graph, eager=r_eager)[schedule]
    p0 = wl.probs[0]
    cold = summarize(r_cold)
    out = dict(step_ms=1e3 * r["wall_s"] / steps,
               lookups_per_s=float(np.sum(r["lookups"])) / r["wall_s"],
               lookups_per_step=int(np.mean(r["lookups"])), T=int(p0.T), B=int(p0.B),
               ms_per_step_serial=1e3 * r_serial["wall_s"] / steps,
               ms_per_step_overlap=1e3 * r_over["wall_s"] / steps,
               ms_per_step_graph=1e3 * r_graph["wall_s"] / steps,
               ms_per_step_eager=1e3 * r_eager["wall_s"] / steps,
               **summarize(r_serial),
               roofline=segment_roofline(r_serial, wl.name, tun),
               cold=dict(note="an untimed 1 GiB read before each forward and each backward, "
                              "outside the stage events", fwd_ms=cold["fwd_ms"], bwd_ms=cold["bwd_ms"],
                         fwd_pct_peak=cold["fwd_pct_peak"], bwd_pct_peak=cold["bwd_pct_peak"],
                         bwd_stage_us=cold["bwd_stage_us"],
                         segment_roofline=segment_roofline(r_cold, wl.name, tun)))
    out["overlap_stage_us"] = stage_us(r_over)
    if extras:
        out["adagrad"] = adagrad_summary(wl, steps, warmup, hip)
        out["mean_pooling"] = mean_pooling_summary(wl, steps, warmup, hip)
    return out


def hist_mfma_flops(wl):
    """Matrix-unit work of one forward when the histogram x table path runs:
    2 * B * rows * D per eligible table (fp16, unweighted, rows and D <= 256,
    mean bag length >= the plan's threshold)."""
    from pooling_tbe_forward_amd import tbe
    p = wl.probs[0]
    if p.wdtype != "f16":
        return 0
    t = tbe.tbe_get_tuning(wl.plan)
    if t.hist_mode == 1 or (t.hist_mode == 0 and p.N < t.hist_min_mean_len * p.T * p.B):
        return 0
    flops = 0
    for k in range(p.T):
        if p.rows[k] <= 256 and p.dims[k] <= 256 and not (p.psw is not None and p.weighted[k]):
            flops += 2 * p.B * int(p.rows[k]) * int(p.dims[k])
    return flops


def report_configs(names, steps, warmup, hip, tuning=None):
    """One JSON line per configuration on stderr (stage times, per-pass % of
    peak, every schedule)."""
    import torch
    for name in names:
        wl = Workload(name, nbatches={"prod": 1}.get(name, 3), tuning=tuning)
        line = dict(config=name, tuning=tuning or {}, N=wl.bytes[0]["N"],
                    unique_rows=wl.bytes[0]["unique_rows"],
                    fwd_bytes_min=wl.bytes[0]["fwd_min"],
                    fwd_bytes_lookup=wl.bytes[0]["fwd_lookup"],
                    bwd_bytes_min=wl.bytes[0]["bwd_min"],
                    **measure(wl, steps, warmup, hip, "eager", extras=tuning is None))
        hist_flops = hist_mfma_flops(wl)
        if hist_flops:   # counts x table on the matrix unit (fp16 in, fp32 accumulate)
            tf = hist_flops / (line["fwd_ms"] * 1e-3) / 1e12
            line["mfma_tflops"] = tf
            line["mfma_pct_peak_fp16"] = 100 * tf / PEAK_MFMA_F16_TFLOPS
        print(json.dumps(line), file=sys.stderr, flush=True)
        del wl
        torch.cuda.empty_cache()


def calibrate_copy(reps=5, nbytes=1 << 30):
    """A plain device copy of known size, to scale the byte counters."""
    import torch
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps(dict(copy_bytes=nbytes, reps=reps)))


def _pmc_rows(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    return rows


def _kernel_avg(rows, pattern, counter):
    vals = [float(r["Counter_Value"]) for r in rows
            if re.search(pattern, r["Kernel_Name"]) and r["Counter_Name"] == counter]
    return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)


def summarize_pmc(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, out, command, workload,
                  tuning):
    """Per-launch HBM bytes of the library's kernels from FETCH_SIZE /
    WRITE_SIZE (KiB per dispatch), each scaled by the ratio of a 1 GiB copy's
    known bytes to what the same counter reported for it."""
    copy_pat = r"copyBuffer|direct_copy"
    cf, _ = _kernel_avg(_pmc_rows(copy_fetch_dir), copy_pat, "FETCH_SIZE")
    cw, _ = _kernel_avg(_pmc_rows(copy_write_dir), copy_pat, "WRITE_SIZE")
    gib_kib = float(1 << 20)
    f_scale = gib_kib / cf if cf else None
    w_scale = gib_kib / cw if cw else None
    res = dict(kernel="k_segment", workload=workload, command=command,
               copy_fetch_kib=cf, copy_write_kib=cw, fetch_scale=f_scale, write_scale=w_scale,
               source_sha256_16=source_hash(SEGMENT_SRC), tuning=tuning, kernels={})
    fetch_rows, write_rows = _pmc_rows(fetch_dir), _pmc_rows(write_dir)
    for name, pat in [("k_segment", r"k_segment"), ("k_fwd_gather", r"k_fwd_gather"),
                      ("k_fwd_hist", r"k_fwd_hist"),
                      ("k_onesweep", r"k_onesweep"), ("k_rle", r"k_rle"),
                      ("k_prep", r"k_prep"), ("k_long_combine", r"k_long_combine")]:
        fv, nf = _kernel_avg(fetch_rows, pat, "FETCH_SIZE")
        wv, nw = _kernel_avg(write_rows, pat, "WRITE_SIZE")
        ent = dict(fetch_kib=fv, write_kib=wv, dispatches=[nf, nw])
        if fv is not None and wv is not None and f_scale and w_scale:
            ent["traffic_bytes"] = int((fv * f_scale + wv * w_scale) * 1024)
        res["kernels"][name] = ent
    res["traffic_bytes"] = res["kernels"]["k_segment"].get("traffic_bytes")
    json.dump(res, open(out, "w"), indent=1)
    print(json.dumps(res))


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--batches", type=int, default=4)
    ap.add_argument("--schedule", default="eager", choices=sorted(SCHEDULE_DESC))
    ap.add_argument("--config", default="mixed", choices=sorted(WORKLOAD_DESC))
    ap.add_argument("--secondary", default="uniform",
                    help="workload measured the same way and nested in the line ('' = none)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--report", action="store_true",
                    help="also print per-configuration measurements on stderr")
    ap.add_argument("--report-configs", default="uniform,mixed,hist,stress,band,prod")
    ap.add_argument("--tau", type=int, default=0, help="long-run threshold for --report")
    ap.add_argument("--chunk", type=int, default=0, help="long-run chunk for --report")
    ap.add_argument("--quick", action="store_true",
                    help="the headline workload's eager steps only (for profilers)")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH", "WRITE", "COPYF", "COPYW"))
    ap.add_argument("--pmc-workload", default="mixed")
    ap.add_argument("--pmc-command", default="")
    ap.add_argument("--pmc-log", default="",
                    help="stdout of the profiled --quick run (its launch knobs)")
    args = ap.parse_args()
    if args.summarize_pmc:
        tuning = None
        if args.pmc_log:
            for line in open(args.pmc_log):
                if line.startswith("{") and '"tuning"' in line:
                    tuning = json.loads(line)["tuning"]
        summarize_pmc(*args.summarize_pmc, traffic_file(args.pmc_workload), args.pmc_command,
                      args.pmc_workload, tuning)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this operator's hot path runs on a single "
              "MI355X here (sharding across GPUs is described, not built); use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from pooling_tbe_forward_amd import tbe
    if not os.path.exists(tbe.LIB_PATH):
        from pooling_tbe_forward_amd import build
        build.build()
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy()
        return
    hip = Hip()
    tuning = {k: v for k, v in (("tau", args.tau), ("chunk", args.chunk)) if v}

    if args.report:
        report_configs([c for c in args.report_configs.split(",") if c], max(10, args.steps // 2),
                       3, hip, tuning or None)
        return

    wl = Workload(args.config, nbatches=args.batches, tuning=tuning or None)
    if args.quick:
        r = run_plain_steps(wl, args.steps, args.warmup)
        print(json.dumps(dict(config=args.config, steps=args.steps,
                              ms_per_step=1e3 * r["wall_s"] / args.steps,
                              tuning=plan_tuning(wl.plan))), flush=True)
        return
    m = measure(wl, args.steps, args.warmup, hip, args.schedule)
    probs = wl.probs
    p0 = probs[0]
    out = dict(metric="TBE fwd/bwd lookups/s and achieved HBM GB/s (% of peak) on 1 MI355X",
               value=m.pop("lookups_per_s"), unit="lookups/s", n_gpus=1, steps=args.steps,
               warmup=args.warmup, ms_per_step=m.pop("step_ms"), higher_is_better=True,
               scaling="weak", vs_baseline=None,
               dtype="f16 weights, f32 accumulate" if p0.wdtype == "f16" else "f32",
               data="synthetic",
               config=dict(workload=WORKLOAD_DESC[args.config], T=m.pop("T"), B=m.pop("B"),
                           lookups_per_step=m.pop("lookups_per_step"),
                           batches_cycled=args.batches, index_dtype="int32",
                           weight_dtype=p0.wdtype, parallelism="single GPU"),
               schedule=SCHEDULE_DESC[args.schedule], **m)
    del wl
    torch.cuda.empty_cache()
    out["int64_indices"] = int64_summary(args.config, probs, args.steps, args.warmup, hip)
    del probs
    if args.secondary:
        wl2 = Workload(args.secondary, nbatches=args.batches)
        m2 = measure(wl2, args.steps, args.warmup, hip, args.schedule, extras=False)
        m2["workload"] = WORKLOAD_DESC[args.secondary]
        out[args.secondary] = m2
        del wl2
        torch.cuda.empty_cache()
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(args.config, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
