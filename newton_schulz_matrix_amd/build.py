"""Build the gfx950 shared library libnsmi.so in-tree with hipcc.

Every source is compiled to an object (in parallel) and the objects are
linked into _lib/libnsmi.so. build() always recompiles every source.

Usage: python -m newton_schulz_matrix_amd.build   (or build() from Python)
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_lib")
OBJ_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "libnsmi.so")
SOURCES = ["ns_api.hip", "norm_kernels.hip", "gemm_kernels.hip"]
ARCH = "gfx950"

COMPILE_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    f"--offload-arch={ARCH}",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
LINK_FLAGS = ["-shared", "-fPIC", f"--offload-arch={ARCH}"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd)}")


def compile_one(src: str, verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    _run([hipcc(), *COMPILE_FLAGS, "-c", os.path.join(SRC, src), "-o", obj], verbose)
    return obj


def link(objs, verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    tmp = LIB + ".tmp"
    _run([hipcc(), *LINK_FLAGS, *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link _lib/libnsmi.so; return its path."""
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: compile_one(s, verbose), SOURCES))
    return link(objs, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
