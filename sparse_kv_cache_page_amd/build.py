"""Build libentmaxkv.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m sparse_kv_cache_page_amd.build        # or build() from Python
    python -m sparse_kv_cache_page_amd.build --incremental   # changed sources only

Each source is compiled by hipcc to an object next to the package's _build/
folder, then linked into sparse_kv_cache_page_amd/libentmaxkv.so.  Packed-fp32
instruction selection is disabled (the kernels are written against the plain
fp32 and fp64 vector units).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libentmaxkv.so")
ARCH = os.environ.get("EKV_OFFLOAD_ARCH", "gfx950")

SOURCES = ["abi.cpp", "meta.hip", "score.hip", "select.hip", "decode.hip", "softmax.hip",
           "noalloc.hip", "step.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-warning-option",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _deps(src: str):
    """The source and the local headers it includes, transitively."""
    import re
    todo, seen = [os.path.join(CSRC, src)], []
    while todo:
        path = todo.pop()
        if path in seen or not os.path.exists(path):
            continue
        seen.append(path)
        with open(path) as fh:
            for name in re.findall(r'^#include "([^"]+)"', fh.read(), flags=re.M):
                todo += [os.path.join(d, name) for d in (CSRC, INCLUDE)]
    return seen


def _compile(src: str, incremental: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    if incremental and os.path.exists(obj):
        t = os.path.getmtime(obj)
        if all(os.path.getmtime(p) < t for p in _deps(src) + [os.path.abspath(__file__)]):
            return obj
    cmd = [hipcc(), *COMMON_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compile every source (incremental: only those whose object is older than
    the source or a local header it includes) and link the library."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda src: _compile(src, incremental), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, incremental="--incremental" in sys.argv[1:])
    sys.exit(0)
