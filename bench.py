#!/usr/bin/env python
"""Benchmark of the TBE hot path on one MI355X: one step = forward pooled sum
+ backward with exact SGD over one batch of the uniform workload (8 tables x
1M rows x D=128 fp32, B=2048, Poisson(20) bags, uniform ids).

Prints ONE JSON line on stdout.  Inputs are resident in HBM before the timed
region; consecutive steps cycle through several distinct batches over the
same tables so that no step re-reads the rows of the step before it from
cache.  `--report` additionally prints per-configuration measurements of the
forward and the backward (one JSON line each) on stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0

WORKLOAD_DESC = {
    "uniform": "uniform TBE: T=8 tables x 1,000,000 rows, D=128 fp32, B=2048, "
               "Poisson(20) bags, uniform ids, unweighted, forward + backward exact SGD",
    "mixed": "mixed TBE: T=40 features, rows log-uniform 1e4..1e7, D in {64,128,256} fp16, "
             "B=4096, geometric(30) bags capped at 500, Zipf(1.1) ids, 20 weighted features",
    "hist": "small-table TBE: T=1 x 64 rows, D=128 fp16, B=16384, 256 ids per bag",
    "stress": "run-length stress TBE: T=4 x 1,000,000 rows, D=128 fp32, B=8192, 50 Zipf(1.2) "
              "ids per bag, weighted",
    "toy": "toy TBE: T=3, rows {100,50,20}, D {8,16,4}, B=4",
}


def algorithmic_bytes(prob):
    """Bytes the method must move (index type int32)."""
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
    bits = max(1, int(np.ceil(np.log2(max(2, int(prob.rows.sum()))))))
    passes = (bits + 7) // 8
    sort_bytes = passes * N * 16 + passes * N * 4
    run_bytes = uk.size * 12
    return dict(N=N, unique_rows=int(uk.size), passes=passes,
                fwd_min=jag + uniq_row_bytes + out_bytes,
                fwd_lookup=jag + lookup_row_bytes + out_bytes,
                bwd_min=jag + out_bytes + 2 * uniq_row_bytes + sort_bytes + run_bytes,
                bwd_rows=2 * uniq_row_bytes)


class Workload:
    """Device-resident inputs for several batches over one set of tables."""

    def __init__(self, name, nbatches, index_dtype="i32"):
        import torch
        from pooling_tbe_forward_amd import datagen as dg
        from pooling_tbe_forward_amd import tbe
        self.name = name
        self.probs = [dg.make_problem(name, batch=k) for k in range(nbatches)]
        p0 = self.probs[0]
        self.weights = dg.packed_weights_torch(p0, "cuda")
        self.plan = tbe.tbe_plan_create(p0.rows, p0.dims,
                                        tbe.TBE_F32 if p0.wdtype == "f32" else tbe.TBE_F16,
                                        tbe.TBE_I32 if index_dtype == "i32" else tbe.TBE_I64,
                                        weighted=p0.weighted)
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
        self.bytes = [algorithmic_bytes(p) for p in self.probs]
        torch.cuda.synchronize()

    def fwd(self, k):
        from pooling_tbe_forward_amd import tbe
        p, d = self.probs[k], self.inputs[k]
        tbe.tbe_forward(self.plan, p.B, self.weights, d["indices"], d["offsets"], d["psw"],
                        self.out)

    def bwd(self, k):
        from pooling_tbe_forward_amd import tbe
        p, d = self.probs[k], self.inputs[k]
        tbe.tbe_backward_sgd(self.plan, p.B, self.weights, d["indices"], d["offsets"], d["psw"],
                             d["grad"], p.lr, self.ws)


def run_steps(wl, steps, warmup, do_fwd=True, do_bwd=True):
    """Warm up, then time `steps` steps; per-step HIP events on the stream the
    library launches on (torch's current stream)."""
    import torch
    nb = len(wl.probs)
    for s in range(warmup):
        if do_fwd:
            wl.fwd(s % nb)
        if do_bwd:
            wl.bwd(s % nb)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        k = s % nb
        ev[s][0].record()
        if do_fwd:
            wl.fwd(k)
        ev[s][1].record()
        if do_bwd:
            wl.bwd(k)
        ev[s][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    f_ms = np.array([ev[s][0].elapsed_time(ev[s][1]) for s in range(steps)])
    b_ms = np.array([ev[s][1].elapsed_time(ev[s][2]) for s in range(steps)])
    ks = [s % nb for s in range(steps)]
    n = np.array([wl.bytes[k]["N"] for k in ks], dtype=np.float64)
    fb = np.array([wl.bytes[k]["fwd_min"] for k in ks], dtype=np.float64)
    bb = np.array([wl.bytes[k]["bwd_min"] for k in ks], dtype=np.float64)
    return dict(wall_s=wall, fwd_ms=f_ms, bwd_ms=b_ms, lookups=n, fwd_bytes=fb, bwd_bytes=bb)


def cpu_baseline(budget_s=20.0):
    """The CPU oracle, as it stands, on the uniform workload's batch 0:
    forward of every bag, the integer stage, and backward-SGD of every touched
    row (rows are regenerated on the host for the touched ids only; that set-up
    is not timed).  Repeated while within the time budget."""
    import oracle
    from pooling_tbe_forward_amd import datagen as dg
    prob = dg.make_problem("uniform")
    rowsets = []
    for t in range(prob.T):
        s, e = prob.offsets[t * prob.B], prob.offsets[(t + 1) * prob.B]
        rowsets.append(np.unique(prob.indices[s:e]))
    tabs = [(ids, np.ascontiguousarray(dg.weight_rows(prob, t, ids).reshape(-1)))
            for t, ids in enumerate(rowsets)]
    code = oracle.F32
    reps, total = 0, 0.0
    stage = dict(forward=0.0, sort_rle=0.0, backward=0.0)
    while total < budget_s and reps < 50:
        t0 = time.perf_counter()
        oracle.forward(prob.T, prob.B, prob.rows, prob.dims, code, tabs, prob.indices,
                       prob.offsets, prob.psw, prob.weighted)
        t1 = time.perf_counter()
        r = oracle.sort_rle(prob.T, prob.B, prob.rows, prob.indices, prob.offsets, 256)
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
    cpu = platform.processor() or platform.machine()
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return dict(value=prob.N * reps / total, unit="lookups/s", cores=1, kind="oracle",
                sample=f"full uniform step (forward all {prob.T * prob.B} bags, sort+RLE of "
                       f"{prob.N} lookups, backward-SGD of every touched row), batch 0, "
                       f"{reps} repetition(s), single thread, fp64 accumulation",
                ms_per_step=1e3 * total / reps,
                stage_ms={k: 1e3 * v / reps for k, v in stage.items()},
                host_cpu=cpu, host_threads=os.cpu_count())


def report_configs(steps, warmup):
    import torch
    for name in ("uniform", "mixed", "hist", "stress"):
        wl = Workload(name, nbatches=3 if name != "mixed" else 2)
        r = run_steps(wl, steps, warmup)
        b = wl.bytes[0]
        f = float(np.median(r["fwd_ms"]))
        g = float(np.median(r["bwd_ms"]))
        line = dict(config=name, N=b["N"], unique_rows=b["unique_rows"],
                    fwd_ms=f, bwd_ms=g,
                    fwd_lookups_per_s=float(np.mean(r["lookups"]) / (f * 1e-3)),
                    bwd_lookups_per_s=float(np.mean(r["lookups"]) / (g * 1e-3)),
                    fwd_gbps_min=float(np.mean(r["fwd_bytes"]) / (f * 1e-3) / 1e9),
                    bwd_gbps_min=float(np.mean(r["bwd_bytes"]) / (g * 1e-3) / 1e9),
                    fwd_bytes_min=b["fwd_min"], fwd_bytes_lookup=b["fwd_lookup"],
                    bwd_bytes_min=b["bwd_min"])
        line["fwd_pct_peak"] = 100 * line["fwd_gbps_min"] / PEAK_HBM_GBPS
        line["bwd_pct_peak"] = 100 * line["bwd_gbps_min"] / PEAK_HBM_GBPS
        print(json.dumps(line), file=sys.stderr, flush=True)
        del wl
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--batches", type=int, default=4)
    ap.add_argument("--config", default="uniform", choices=sorted(WORKLOAD_DESC))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--report", action="store_true",
                    help="also print per-configuration fwd/bwd measurements on stderr")
    args = ap.parse_args()
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

    wl = Workload(args.config, nbatches=args.batches)
    r = run_steps(wl, args.steps, args.warmup)
    step_ms = 1e3 * r["wall_s"] / args.steps
    lookups = float(np.sum(r["lookups"]))
    value = lookups / r["wall_s"]
    f_ms = float(np.mean(r["fwd_ms"]))
    b_ms = float(np.mean(r["bwd_ms"]))
    f_gbps = float(np.mean(r["fwd_bytes"])) / (f_ms * 1e-3) / 1e9
    b_gbps = float(np.mean(r["bwd_bytes"])) / (b_ms * 1e-3) / 1e9
    p0 = wl.probs[0]
    # Dominant kernel: the forward gather (one launch per tbe_forward on this
    # workload); its algorithmic bytes per launch are the forward's B_min.
    roof = dict(bound="hbm", kernel="k_fwd_gather", achieved=round(f_gbps, 1),
                peak=PEAK_HBM_GBPS, unit="GB/s", frac=round(f_gbps / PEAK_HBM_GBPS, 4),
                traffic=None, avg_launch_us=round(1e3 * f_ms, 2),
                bytes_per_launch=int(np.mean(r["fwd_bytes"])))
    out = dict(metric="TBE fwd/bwd lookups/s and achieved HBM GB/s (% of peak) on 1 MI355X",
               value=value, unit="lookups/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
               ms_per_step=step_ms, higher_is_better=True, scaling="weak", vs_baseline=None,
               dtype="f32", data="synthetic",
               config=dict(workload=WORKLOAD_DESC[args.config], T=int(p0.T), B=int(p0.B),
                           lookups_per_step=int(np.mean(r["lookups"])),
                           batches_cycled=args.batches, index_dtype="int32",
                           bwd_accumulation="f64", parallelism="single GPU"),
               fwd_ms=f_ms, bwd_ms=b_ms,
               fwd_lookups_per_s=float(np.mean(r["lookups"])) / (f_ms * 1e-3),
               bwd_lookups_per_s=float(np.mean(r["lookups"])) / (b_ms * 1e-3),
               fwd_hbm_gbps_min=f_gbps, bwd_hbm_gbps_min=b_gbps,
               fwd_pct_peak=100 * f_gbps / PEAK_HBM_GBPS,
               bwd_pct_peak=100 * b_gbps / PEAK_HBM_GBPS,
               roofline=roof)
    del wl
    torch.cuda.empty_cache()
    if args.report:
        report_configs(max(10, args.steps // 2), 3)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
