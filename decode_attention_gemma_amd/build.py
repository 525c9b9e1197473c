"""Build libg4attn.so (HIP kernels + C-ABI host code) for gfx950, in-tree,
and libg4probe.so, the hardware-rate probes bench.py --read-probe and
--gemm-probe use."""

from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libg4attn.so")
PROBE_LIB = os.path.join(HERE, "libg4probe.so")

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
SOURCES = ["kernels.hip", "plan.cpp"]


def hipcc() -> str:
    return os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def build_library(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), *HIP_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        _run(cmd, verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    _run([hipcc(), *HIP_FLAGS, "-shared", "-x", "hip", os.path.join(CSRC, "hw_probes.hip"),
          "-o", tmp], verbose)
    os.replace(tmp, PROBE_LIB)
    return LIB


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n"
                           f"{r.stdout}\n{r.stderr}")


if __name__ == "__main__":
    print(build_library(verbose=True))
