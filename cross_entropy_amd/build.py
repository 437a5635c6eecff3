"""Builds the HIP library ``liblmhead_logps.so`` in-tree for gfx950.

    python -m cross_entropy_amd.build             (from the repository root)
    python -m cross_entropy_amd.build --sanitize  (host ASan + UBSan build)

Every call compiles from source (no cache). The library holds the kernels
and the C ABI of ``include/lmhead_logps.h``; the Python binding loads it
from this directory.

``--sanitize`` builds ``liblmhead_logps_sanitize.so`` with AddressSanitizer
and UndefinedBehaviorSanitizer on the host code only (argument checks, the
planner, workspace layout, tracing; the device code is built as usual). The
host tests run against it with the ASan runtime preloaded and
``LMHEAD_LOGPS_LIB`` pointing the binding at it; ``sanitizer_env()`` gives
that environment.
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


SANITIZE_LIB_PATH = os.path.join(PKG, "liblmhead_logps_sanitize.so")
# host-only sanitizers: each -fsanitize= applies to the host compilation
SANITIZE_FLAGS = [
    "-Xarch_host", "-g", "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
]


def asan_runtime() -> str:
    """The clang ASan runtime matching hipcc's host compiler."""
    out = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        import glob
        found = sorted(glob.glob("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
        if not found:
            raise RuntimeError("libclang_rt.asan-x86_64.so not found")
        path = found[-1]
    return path


def sanitizer_env() -> dict:
    """Environment for a host process that loads the sanitizer build."""
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan_runtime()
    env["LMHEAD_LOGPS_LIB"] = SANITIZE_LIB_PATH
    # the Python interpreter itself is not instrumented; its allocations are
    # not leaks of the library
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return env


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile the library (or its host-sanitized variant) and return its
    path. Raises on failure."""
    out = SANITIZE_LIB_PATH if sanitize else LIB_PATH
    tmp = out + ".tmp"
    flags = HIP_FLAGS + (SANITIZE_FLAGS if sanitize else [])
    cmd = [hipcc()] + flags + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
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
    os.replace(tmp, out)
    return out


CAPI_SRC = os.path.join(ROOT, "tests", "capi", "capi_check.cpp")
CAPI_BIN = os.path.join(ROOT, "tests", "capi", "capi_check")


def build_capi_check(verbose: bool = False) -> str:
    """Compile tests/capi/capi_check.cpp, a caller of the C ABI with no Python
    and no PyTorch, linked against the in-tree library (run by the GPU test
    tests/test_gpu_capi.py). Needs the library built first."""
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build the library first")
    tmp = CAPI_BIN + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-O2", "-std=c++17", "-Wall", CAPI_SRC, "-o", tmp,
           "-L" + PKG, "-llmhead_logps", "-Wl,-rpath,$ORIGIN/../../cross_entropy_amd"]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{proc.stderr}")
    os.replace(tmp, CAPI_BIN)
    return CAPI_BIN


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv[1:]))
