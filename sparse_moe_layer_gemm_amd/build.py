"""Build the HIP library liblatentmoe.so (gfx950) in-tree with hipcc, and the
benchmark's HBM read yardstick libhbmread.so."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "latentmoe.hip")
LIB = os.path.join(PKG, "liblatentmoe.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep the compiler from forming packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# the benchmark's HBM streaming-read yardstick (not part of the layer)
PROBE_SRC = os.path.join(PKG, "csrc", "hbm_read.hip")
PROBE_LIB = os.path.join(PKG, "libhbmread.so")


def _hipcc(src: str, lib: str, verbose: bool) -> None:
    cmd = [hipcc(), *HIPCC_FLAGS, src, "-o", lib + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(lib)}")
    os.replace(lib + ".tmp", lib)


def build(verbose: bool = False) -> str:
    _hipcc(SRC, LIB, verbose)
    _hipcc(PROBE_SRC, PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
