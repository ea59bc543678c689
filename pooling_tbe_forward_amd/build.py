"""Build libtbe.so (HIP, gfx950) in-tree with hipcc, and beside it
libtbe_datagen.so, the device half of the seeded input generator (test and
benchmark inputs only; it holds none of the operator's arithmetic).

Usage: python -m pooling_tbe_forward_amd.build [--jobs N]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libtbe.so")
GEN_SRC = os.path.join(HERE, "gen", "weights_gen.hip")
GEN_LIB = os.path.join(HERE, "libtbe_datagen.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["tbe_api.hip", "fwd_gather.hip", "fwd_hist.hip", "bwd_sort.hip", "bwd_segment.hip",
           "bounds_check.hip"]

# Packed-fp32 VALU ops are disabled: the compiler may still use scalar and
# float2 code, but never emits v_pk_{add,mul,fma}_f32.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-result"]


def _compile(src: str) -> str:
    os.makedirs(BUILD, exist_ok=True)
    path = src if os.path.isabs(src) else os.path.join(CSRC, src)
    obj = os.path.join(BUILD, os.path.splitext(os.path.basename(src))[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(jobs: int = 8, verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libtbe.so and
    libtbe_datagen.so (always rebuilds)."""
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES + [GEN_SRC]))
    _link(objs[:-1], LIB)
    _link(objs[-1:], GEN_LIB)
    if verbose:
        print("built", LIB, "and", GEN_LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    args = ap.parse_args()
    build(args.jobs, verbose=True)
    sys.exit(0)
