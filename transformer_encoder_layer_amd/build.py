"""Ahead-of-time build of libtel.so (gfx950) from the HIP sources in csrc/,
and of libtel_debug.so: the same objects except the C ABI (tel_api.hip),
compiled with TEL_DEBUG_CHECKS so that every forward and backward checks the
device key lengths on the host.

Usage: python -m transformer_encoder_layer_amd.build   (or build() from Python)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libtel.so")
OUT_DEBUG = os.path.join(HERE, "libtel_debug.so")
BUILD = os.path.join(HERE, "_build")
ROOT = os.path.dirname(HERE)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-fno-gpu-rdc",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result", "-I", os.path.join(ROOT, "include")]


# Per-source extra flags.  gemm.hip: the epilogues fully unroll a loop over
# the accumulator blocks around a large per-row body (dropout, GELU); below
# this threshold the unroller gives up and the accumulators are indexed
# dynamically, i.e. moved to scratch memory.
EXTRA = {"gemm.hip": ["-mllvm", "-pragma-unroll-threshold=200000"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


DEBUG_SRC = "tel_api.hip"


def _compile(job) -> str:
    src, debug = job
    base = os.path.basename(src)[:-4] + ("_debug" if debug else "")
    obj = os.path.join(BUILD, base + ".o")
    defs = ["-DTEL_DEBUG_CHECKS"] if debug else []
    cmd = [HIPCC, *FLAGS, *defs, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fno-gpu-rdc", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    # the largest source first, so the pool's critical path is its compile
    jobs = sorted([(s, False) for s in srcs], key=lambda j: -os.path.getsize(j[0]))
    jobs.append((os.path.join(CSRC, DEBUG_SRC), True))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = dict(zip(jobs, ex.map(_compile, jobs)))
    release = [objs[(s, False)] for s in srcs]
    debug = [objs[(s, os.path.basename(s) == DEBUG_SRC)] for s in srcs]
    _link(release, OUT)
    _link(debug, OUT_DEBUG)
    if verbose:
        print(f"built {OUT} and {OUT_DEBUG}")
    return OUT


if __name__ == "__main__":
    build()
    sys.exit(0)
