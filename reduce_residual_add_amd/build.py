"""Build libtwnorm.so in-tree for gfx950 (hipcc), next to this file.

Usage:  python -m reduce_residual_add_amd.build [-v]
The HIP sources compile in parallel; the HIP-free validator compiles with g++.
Extra preprocessor flags for experiments can be passed through the
TWNORM_EXTRA_FLAGS environment variable (e.g. "-DTW_NT_LOADS=1").
"""
from __future__ import annotations

import os
import shlex
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtwnorm.so")

HIP_SOURCES = ["twnorm_api.hip", "twnorm_fused_bf16.hip", "twnorm_fused_f32.hip"]
CPP_SOURCES = ["twnorm_validate.cpp"]

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed-fp32 VALU forms stay disabled: only scalar/float2 code the
# compiler vectorises itself would use them, and they are not needed here.
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I" + INCLUDE, "-I" + CSRC]
CPP_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I" + INCLUDE, "-I" + CSRC]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(shlex.quote(c) for c in cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    if verbose and out:
        print(out)
    return r


def build(verbose: bool = False) -> str:
    """Compile every source and link libtwnorm.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    extra = shlex.split(os.environ.get("TWNORM_EXTRA_FLAGS", ""))
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        jobs.append([HIPCC, *HIP_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in CPP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        jobs.append(["g++", *CPP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    workers = min(len(jobs), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    p = build(verbose="-v" in sys.argv)
    print(p)
