"""Build the HIP library (gfx950) in-tree with hipcc.

The product is ``libsinkhorn.so`` next to this file; its C ABI is declared in
``include/sinkhorn.h`` at the repository root.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
SRC = os.path.join(PKG_DIR, "csrc", "sinkhorn.hip")
PEAKS_SRC = os.path.join(PKG_DIR, "csrc", "peaks.hip")
PEAKS_LIB = os.path.join(PKG_DIR, "libskpeaks.so")
INC = os.path.join(ROOT, "include")
LIB = os.path.join(PKG_DIR, "libsinkhorn.so")
ARCH = os.environ.get("SINKHORN_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3",
    f"--offload-arch={ARCH}",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build_library(verbose: bool = False) -> str:
    """Compile csrc/sinkhorn.hip into libsinkhorn.so (always recompiles)."""
    return _hipcc(SRC, LIB, verbose)


def build_peaks(verbose: bool = False) -> str:
    """Compile the peak-rate microbenchmarks csrc/peaks.hip into libskpeaks.so."""
    return _hipcc(PEAKS_SRC, PEAKS_LIB, verbose)


def _hipcc(src: str, lib: str, verbose: bool) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = lib + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, f"-I{INC}", src, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build_library(verbose=True))
    print(build_peaks(verbose=True))
