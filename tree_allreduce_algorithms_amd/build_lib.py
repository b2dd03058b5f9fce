"""Build libar.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Usage: ``python -m tree_allreduce_algorithms_amd.build_lib`` (or call
``build()``).  hipcc cross-compiles for gfx950 without a GPU present.  Each
source compiles to its own object in parallel (the kernel files instantiate
many dtype x op x unroll variants), then one hipcc call links the library.
"""

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libar.so")

SOURCES = ["api.cpp", "plan.cpp", "ring_kernels.hip", "copy_kernels.hip", "tree_kernels.hip",
           "step_kernels.hip"]

COMPILE_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # one IEEE operation per hop: no contraction, no flushing of subnormals
    "-ffp-contract=off",
    "-fno-gpu-flush-denormals-to-zero",
    # keep the compiler from emitting packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]
LINK_FLAGS = ["--offload-arch=gfx950", "-shared", "-fPIC"]


def hipcc():
    exe = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError(f"hipcc not found (looked for {exe})")
    return exe


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose=False, jobs=None):
    """Compile every source into libar.so next to this file; returns its path."""
    cc = hipcc()
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 8)
    with tempfile.TemporaryDirectory(prefix="ar_build_") as tmpdir:
        objs, procs, pending = [], [], list(sources())
        failures = []
        while pending or procs:
            while pending and len(procs) < jobs:
                src = pending.pop(0)
                obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
                cmd = [cc, *COMPILE_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
                if verbose:
                    print(" ".join(cmd), flush=True)
                procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                    stderr=subprocess.STDOUT, text=True)))
                objs.append(obj)
            src, proc = procs.pop(0)
            out, _ = proc.communicate()
            if proc.returncode != 0:
                failures.append(f"{os.path.basename(src)} ({proc.returncode}):\n{out}")
            elif verbose and out.strip():
                print(out, file=sys.stderr)
        if failures:
            raise RuntimeError("hipcc failed:\n" + "\n".join(failures))
        tmp = LIB + ".tmp"
        cmd = [cc, *LINK_FLAGS, *objs, "-o", tmp]
        proc = subprocess.run(cmd, capture_output=True, text=True)
        if proc.returncode != 0:
            raise RuntimeError(f"link failed ({proc.returncode}):\n{proc.stdout}\n{proc.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
