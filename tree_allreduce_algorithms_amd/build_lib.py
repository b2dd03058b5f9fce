"""Build libar.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Usage: ``python -m tree_allreduce_algorithms_amd.build_lib`` (or call
``build()``).  hipcc cross-compiles for gfx950 without a GPU present.
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libar.so")

SOURCES = ["api.cpp", "plan.cpp", "kernels.hip"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # one IEEE operation per hop: no contraction, no flushing of subnormals
    "-ffp-contract=off",
    "-fno-gpu-flush-denormals-to-zero",
    # keep the compiler from emitting packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc():
    exe = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError(f"hipcc not found (looked for {exe})")
    return exe


def build(verbose=False):
    """Compile every source into libar.so next to this file; returns its path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{proc.stdout}\n{proc.stderr}")
    if verbose and proc.stderr.strip():
        print(proc.stderr, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
