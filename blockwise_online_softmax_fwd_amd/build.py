"""Build libringattn.so for gfx950 with hipcc (in-tree, no JIT cache).

Every HIP source is compiled for gfx950 only; the shared library lands next to
this file, where the Python binding loads it.  Packed fp32 VALU instructions
are switched off for all device code.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libringattn.so")

SOURCES = ["api.cpp", "classify.hip", "attn_bf16.hip", "attn_f32.hip", "merge.hip", "reorder.hip",
           "bwd.hip"]

# Per-source code generation options (none at present).
EXTRA_FLAGS: dict = {}

ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libringattn)")


def common_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
        "-Wall", "-Wno-unused-function",
    ]


def _compile(src: str, verbose: bool) -> str:
    out = os.path.join(BUILD, src + ".o")
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", out] + common_flags() + EXTRA_FLAGS.get(src, [])
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(min(len(SOURCES), max(1, os.cpu_count() or 1))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
