"""Build the gfx950 HIP library ``libdash.so`` in-tree with hipcc.

    python sparse_hierarchical_attention_block_amd/build.py [--incremental]

Every HIP source is compiled for gfx950 only, with packed-FP32 instruction
selection disabled, then linked into one shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build", "dash")
LIB = os.path.join(PKG, "libdash.so")
SOURCES = ["summarize.hip", "route.hip", "route_tile.hip", "route_long.hip", "attend.hip",
           "decode.hip", "backward.hip", "peaks.hip", "api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _headers_mtime() -> float:
    hdrs = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hpp", ".h"))]
    hdrs.append(os.path.join(ROOT, "include", "dash.h"))
    return max(os.path.getmtime(h) for h in hdrs)


def _compile(src: str, incremental: bool = False) -> str:
    out = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    if incremental and os.path.exists(out):
        newest = max(os.path.getmtime(os.path.join(CSRC, src)), _headers_mtime(),
                     os.path.getmtime(os.path.abspath(__file__)))
        if os.path.getmtime(out) > newest:
            return out
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return out


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compile every source (incremental: only those older than their .o or
    any header) and link libdash.so."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, incremental), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "--offload-arch=gfx950", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB, file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True, incremental="--incremental" in sys.argv)
