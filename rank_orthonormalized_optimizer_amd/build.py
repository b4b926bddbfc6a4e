"""Build the gfx950 shared library ``libdion_mi355x.so`` in-tree with hipcc.

Run ``python -m rank_orthonormalized_optimizer_amd.build`` (or call ``build()``).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libdion_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["dion_step.hip", "stream16.hip", "elementwise.hip", "spectral.hip", "noalloc.hip", "dion_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    cand = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def compile_flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # never emit packed-fp32 instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Wall", "-Wno-unused-function",
    ]


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    objs = []
    os.makedirs(os.path.join(HERE, "_build"), exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(HERE, "_build", src + ".o")
        lang = [] if src.endswith(".hip") else ["-x", "hip"]
        cmd = [hipcc()] + compile_flags() + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
