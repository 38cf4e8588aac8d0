"""Builds libdyra.so in-tree for gfx950 (hipcc for the HIP sources, g++ for the host factorisation)."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
OUT = os.path.join(PKG, "libdyra.so")
BUILD = os.path.join(ROOT, "_build")

HIP_SOURCES = ["dyra_api.hip", "gemm.hip", "solve.hip", "dyra_decode.hip", "als.hip", "ns.hip", "blast.hip"]
CXX_SOURCES = ["host_factorize.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 instructions are kept out of every kernel.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-result", "-I", os.path.join(ROOT, "include")]
CXX_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-fopenmp", "-march=x86-64-v2", "-I", os.path.join(ROOT, "include")]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout)
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}")
    return r.stdout


def build(verbose: bool = False) -> str:
    """Compiles every source and links libdyra.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(["g++", *CXX_FLAGS], src) for src in CXX_SOURCES] + [([HIPCC, *HIP_FLAGS], src) for src in HIP_SOURCES]
    objs = [os.path.join(BUILD, src + ".o") for _, src in jobs]

    def compile_one(job):
        (cc, src), obj = job
        return _run([*cc, "-c", os.path.join(CSRC, src), "-o", obj])

    # the sources compile independently: one compiler process per source
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        for out in pool.map(compile_one, zip(jobs, objs)):
            if verbose and out.strip():
                print(out)
    tmp = OUT + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, "-lgomp"])
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
