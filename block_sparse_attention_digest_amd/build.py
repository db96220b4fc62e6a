"""Build libscoutattn.so for gfx950 with hipcc (objects in parallel, then one link).

The HIP sources go through hipcc; the host-only C++ source (the CPU partial attention) goes
through the host C++ compiler, which can give it per-CPU clones.

    python -m block_sparse_attention_digest_amd.build

The library lands next to this file; objects go to _build/ (not committed).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libscoutattn.so")

SOURCES = ["api.hip", "layout.hip", "digest.hip", "gemm.hip", "select.hip", "attention.hip",
           "recall.hip", "dense.hip", "handoff.hip", "host_attention.cpp", "host_handoff.cpp"]
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-result",
    # packed-FP32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
]


# -Wno-psabi: the 32-byte vector helpers are internal, so their calling convention never
# crosses an interface
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-psabi", "-pthread", f"-I{INCLUDE}"]


def host_cxx() -> str:
    for c in (os.environ.get("CXX"), shutil.which("g++"), shutil.which("c++")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("no host C++ compiler found (g++ is required to build libscoutattn)")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libscoutattn)")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libscoutattn.so; returns its path."""
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        if src.endswith(".hip"):
            jobs.append([cc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        else:
            jobs.append([host_cxx(), *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        for msg in ex.map(_run, jobs):
            if msg.strip() and verbose:
                print(msg, file=sys.stderr)
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
