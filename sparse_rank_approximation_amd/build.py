"""Builds libelsaa.so (the gfx950 HIP kernels and their C ABI) in-tree with hipcc.

    python -m sparse_rank_approximation_amd.build [--force]

Every source is compiled to an object under _build/ in parallel, then linked
into sparse_rank_approximation_amd/libelsaa.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libelsaa.so")
SOURCES = ["select.hip", "lowrank.hip", "fwd.hip", "bwd.hip", "merge.hip", "gates.hip", "topk.hip",
           "extra.hip", "check.hip", "fused.hip", "api.cpp", "prof.cpp"]
HEADERS = ["common.hpp", "launch.hpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}",
         # Packed fp32 instructions stay off in the device code.
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile every source and link libelsaa.so. With force=False sources older
    than the library are not recompiled."""
    os.makedirs(BUILD, exist_ok=True)
    deps = [os.path.join(CSRC, h) for h in HEADERS] + [os.path.join(INCLUDE, "elsaa.h")]
    newest_dep = max(os.path.getmtime(p) for p in deps)
    todo = []
    for s in SOURCES:
        obj = os.path.join(BUILD, s + ".o")
        if force or not os.path.exists(obj) or os.path.getmtime(obj) < max(
                os.path.getmtime(os.path.join(CSRC, s)), newest_dep):
            todo.append(s)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        for obj in ex.map(_compile, todo):
            if verbose:
                print("compiled", os.path.relpath(obj, ROOT), flush=True)
    objs = [os.path.join(BUILD, s + ".o") for s in SOURCES]
    tmp = LIB + f".tmp{os.getpid()}"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--force" in sys.argv or True, verbose=True))
