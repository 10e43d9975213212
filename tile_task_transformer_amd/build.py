"""Builds libtiletask.so for gfx950 in-tree with hipcc.

Usage: python tile_task_transformer_amd/build.py [--jobs N] [--debug]

Each source under csrc/ compiles to an object (in parallel), then hipcc
links the shared library next to this file. Every compile disables packed
fp32 instructions (hipcc otherwise forms v_pk_*_f32 from float code).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtiletask.so")
ARCH = os.environ.get("TT_OFFLOAD_ARCH", "gfx950")

SOURCES = ["runtime.cpp", "tasks.cpp", "gpt2.cpp", "gemm.hip", "layernorm.hip", "softmax.hip", "attention.hip", "misc.hip",
           "probe.hip", "rope_swiglu.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtiletask)")


def flags(debug: bool):
    f = ["-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-function",
         "-Wno-unused-result"]
    f += ["-O1", "-g"] if debug else ["-O3"]
    return f


def compile_one(src: str, debug: bool) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(OBJ, src + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc()] + flags(debug) + lang + ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 0, debug: bool = False, verbose: bool = True) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: compile_one(s, debug), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--debug", action="store_true")
    a = ap.parse_args(argv)
    build(a.jobs, a.debug)


if __name__ == "__main__":
    sys.exit(main())
