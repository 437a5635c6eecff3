"""Builds the HIP library ``liblmhead_logps.so`` in-tree for gfx950.

    python -m cross_entropy_amd.build        (from the repository root)

Every call compiles from source (no cache). The library holds the kernels
and the C ABI of ``include/lmhead_logps.h``; the Python binding loads it
from this directory.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_NAME = "liblmhead_logps.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["lmhead_api.hip", "lmhead_kernels.hip", "lmhead_trace.hip"]
HEADERS = ["lmhead_internal.h", os.path.join("..", "..", "include", "lmhead_logps.h")]

# Packed-fp32 VALU ops are kept out of the generated code on purpose.
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def build(verbose: bool = False) -> str:
    """Compile the library and return its path. Raises on failure."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc()] + HIP_FLAGS + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature and says so
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in proc.stderr.splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
