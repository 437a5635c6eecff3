"""ctypes binding of the C ABI in ``include/lmhead_logps.h``.

Argument marshalling only: every step of the head runs in the HIP library.
There is no CPU fallback; loading fails loudly when the library is missing.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# LMHEAD_LOGPS_LIB names another build of the library to load (the host
# sanitizer build of cross_entropy_amd/build.py --sanitize)
LIB_PATH = os.environ.get("LMHEAD_LOGPS_LIB") or os.path.join(_PKG, "liblmhead_logps.so")

LMH_OK = 0
ERROR_NAMES = {
    -1: "LMH_ERR_NULL",
    -2: "LMH_ERR_SHAPE",
    -3: "LMH_ERR_CHUNK",
    -4: "LMH_ERR_WORKSPACE",
    -5: "LMH_ERR_ARGS",
    -6: "LMH_ERR_UNSUPPORTED",
    -7: "LMH_ERR_HIP",
}

EXPORTED = (
    "lmhead_logps_workspace_bytes",
    "lmhead_logps_fwd",
    "lmhead_logps_bwd",
    "lmhead_logps_fwd_temp",
    "lmhead_logps_bwd_temp",
    "lmhead_logps_bwd_ex",
    "lmhead_logps_bwd_bf16",
    "lmhead_logps_fwd_shard",
    "lmhead_logps_merge_shards",
    "lmhead_logps_bwd_shard",
    "lmhead_logps_fwd_noalloc",
    "lmhead_logps_last_error",
    "lmhead_logps_version",
    "lmhead_logps_trace_enable",
    "lmhead_logps_trace_read",
    "lmhead_logps_trace_kernel_name",
)


class LmheadError(RuntimeError):
    """A non-zero status from the library, with its name and message."""

    def __init__(self, code: int, message: str):
        self.code = code
        self.name = ERROR_NAMES.get(code, str(code))
        super().__init__(f"{self.name} ({code}): {message}")


_lib = None


def _hip_runtimes_mapped():
    try:
        with open("/proc/self/maps") as f:
            return sorted({l.split()[-1] for l in f if "libamdhip64" in l})
    except OSError:  # pragma: no cover
        return []


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and return the HIP library; raise if it is not built.

    PyTorch is imported first so that the library binds to the HIP runtime
    PyTorch already loaded (its wheel bundles one with the same soname):
    device pointers and streams handed over from torch are only valid in
    that runtime. A process that ends up with two HIP runtimes is refused."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: the HIP library is not built "
            "(run `python -m cross_entropy_amd.build` or __graft_entry__.build())")
    import torch  # noqa: F401  (binds the library to torch's HIP runtime)
    lib = ctypes.CDLL(path)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError(f"two HIP runtimes are loaded in this process: {runtimes}")
    i64, p, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    lib.lmhead_logps_workspace_bytes.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.POINTER(sz)]
    lib.lmhead_logps_workspace_bytes.restype = ctypes.c_int
    lib.lmhead_logps_fwd.argtypes = [p, p, p, i64, i64, i64, i64, p, p, p, p, sz, p]
    lib.lmhead_logps_fwd.restype = ctypes.c_int
    lib.lmhead_logps_bwd.argtypes = [p, p, p, i64, i64, i64, i64, p, p, p, p, p, p, p, sz, p]
    lib.lmhead_logps_bwd.restype = ctypes.c_int
    f32 = ctypes.c_float
    lib.lmhead_logps_fwd_temp.argtypes = [p, p, p, i64, i64, i64, i64, f32, p, p, p, p, sz, p]
    lib.lmhead_logps_fwd_temp.restype = ctypes.c_int
    lib.lmhead_logps_bwd_temp.argtypes = [p, p, p, i64, i64, i64, i64, f32, p, p, p, p, p, p, p, sz, p]
    lib.lmhead_logps_bwd_temp.restype = ctypes.c_int
    lib.lmhead_logps_bwd_ex.argtypes = [p, p, p, i64, i64, i64, i64, f32, p, p, p, p, p, p, ctypes.c_uint, p, sz, p]
    lib.lmhead_logps_bwd_ex.restype = ctypes.c_int
    lib.lmhead_logps_bwd_bf16.argtypes = [p, p, p, i64, i64, i64, i64, f32, p, p, p, p, p, p, ctypes.c_uint, p, sz,
                                          p]
    lib.lmhead_logps_bwd_bf16.restype = ctypes.c_int
    lib.lmhead_logps_fwd_shard.argtypes = [p, p, p, i64, i64, i64, i64, i64, i64, f32, p, p, sz, p]
    lib.lmhead_logps_fwd_shard.restype = ctypes.c_int
    lib.lmhead_logps_merge_shards.argtypes = [p, i64, p, i64, i64, f32, p, p, p, p]
    lib.lmhead_logps_merge_shards.restype = ctypes.c_int
    lib.lmhead_logps_bwd_shard.argtypes = [p, p, p, i64, i64, i64, i64, i64, i64, f32, p, p, p, p, p, p,
                                           ctypes.c_uint, p, sz, p]
    lib.lmhead_logps_bwd_shard.restype = ctypes.c_int
    lib.lmhead_logps_fwd_noalloc.argtypes = [p, p, p, i64, i64, i64, i64, f32, p, p, p, p]
    lib.lmhead_logps_fwd_noalloc.restype = ctypes.c_int
    lib.lmhead_logps_last_error.argtypes = []
    lib.lmhead_logps_last_error.restype = ctypes.c_char_p
    lib.lmhead_logps_version.argtypes = []
    lib.lmhead_logps_version.restype = ctypes.c_char_p
    lib.lmhead_logps_trace_enable.argtypes = [ctypes.c_int]
    lib.lmhead_logps_trace_enable.restype = ctypes.c_int
    dp = ctypes.POINTER(ctypes.c_double)
    lib.lmhead_logps_trace_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int64), dp, dp, dp]
    lib.lmhead_logps_trace_read.restype = ctypes.c_int
    lib.lmhead_logps_trace_kernel_name.argtypes = [ctypes.c_int]
    lib.lmhead_logps_trace_kernel_name.restype = ctypes.c_char_p
    _lib = lib
    return lib


def check(code: int) -> None:
    if code != LMH_OK:
        msg = load().lmhead_logps_last_error().decode(errors="replace")
        raise LmheadError(code, msg)


WS_FWD, WS_BWD, WS_BWD_BF16 = 0, 1, 2


def raw_workspace_bytes(N: int, H: int, V: int, chunk_size: int, with_backward) -> int:
    """with_backward: False / True (WS_FWD / WS_BWD) or WS_BWD_BF16."""
    out = ctypes.c_size_t(0)
    check(load().lmhead_logps_workspace_bytes(int(N), int(H), int(V), int(chunk_size), int(with_backward),
                                              ctypes.byref(out)))
    return int(out.value)


def raw_fwd(hidden, W, targets, N, H, V, chunk_size, logp, entropy, lse, workspace, workspace_bytes,
            stream) -> int:
    """Call lmhead_logps_fwd with integer addresses (0 = NULL); returns the status."""
    return load().lmhead_logps_fwd(hidden or None, W or None, targets or None, int(N), int(H), int(V),
                                   int(chunk_size), logp or None, entropy or None, lse or None,
                                   workspace or None, int(workspace_bytes), stream or None)


def raw_bwd(hidden, W, targets, N, H, V, chunk_size, lse, entropy, g_logp, g_ent, dh, dW, workspace,
            workspace_bytes, stream) -> int:
    """Call lmhead_logps_bwd with integer addresses (0 = NULL); returns the status."""
    return load().lmhead_logps_bwd(hidden or None, W or None, targets or None, int(N), int(H), int(V),
                                   int(chunk_size), lse or None, entropy or None, g_logp or None,
                                   g_ent or None, dh or None, dW or None, workspace or None,
                                   int(workspace_bytes), stream or None)


def raw_fwd_temp(hidden, W, targets, N, H, V, chunk_size, temperature, logp, entropy, lse, workspace,
                 workspace_bytes, stream) -> int:
    """Call lmhead_logps_fwd_temp with integer addresses (0 = NULL); returns the status."""
    return load().lmhead_logps_fwd_temp(hidden or None, W or None, targets or None, int(N), int(H), int(V),
                                        int(chunk_size), float(temperature), logp or None, entropy or None,
                                        lse or None, workspace or None, int(workspace_bytes), stream or None)


def raw_bwd_temp(hidden, W, targets, N, H, V, chunk_size, temperature, lse, entropy, g_logp, g_ent, dh, dW,
                 workspace, workspace_bytes, stream) -> int:
    """Call lmhead_logps_bwd_temp with integer addresses (0 = NULL); returns the status."""
    return load().lmhead_logps_bwd_temp(hidden or None, W or None, targets or None, int(N), int(H), int(V),
                                        int(chunk_size), float(temperature), lse or None, entropy or None,
                                        g_logp or None, g_ent or None, dh or None, dW or None,
                                        workspace or None, int(workspace_bytes), stream or None)


BWD_ACCUMULATE_DH = 1
BWD_ACCUMULATE_DW = 2


def raw_bwd_ex(hidden, W, targets, N, H, V, chunk_size, temperature, lse, entropy, g_logp, g_ent, dh, dW, flags,
               workspace, workspace_bytes, stream) -> int:
    """Call lmhead_logps_bwd_ex with integer addresses (0 = NULL); returns the status."""
    return load().lmhead_logps_bwd_ex(hidden or None, W or None, targets or None, int(N), int(H), int(V),
                                      int(chunk_size), float(temperature), lse or None, entropy or None,
                                      g_logp or None, g_ent or None, dh or None, dW or None, int(flags),
                                      workspace or None, int(workspace_bytes), stream or None)


def raw_bwd_bf16(hidden, W, targets, N, H, V, chunk_size, temperature, lse, entropy, g_logp, g_ent, dh, dW, flags,
                 workspace, workspace_bytes, stream) -> int:
    """Call lmhead_logps_bwd_bf16 with integer addresses (0 = NULL); returns the status."""
    return load().lmhead_logps_bwd_bf16(hidden or None, W or None, targets or None, int(N), int(H), int(V),
                                        int(chunk_size), float(temperature), lse or None, entropy or None,
                                        g_logp or None, g_ent or None, dh or None, dW or None, int(flags),
                                        workspace or None, int(workspace_bytes), stream or None)


def raw_fwd_shard(hidden, W_shard, targets, N, H, V_shard, vocab_offset, V_total, chunk_size, temperature,
                  partial, workspace, workspace_bytes, stream) -> int:
    """Call lmhead_logps_fwd_shard with integer addresses (0 = NULL); returns the status."""
    return load().lmhead_logps_fwd_shard(hidden or None, W_shard or None, targets or None, int(N), int(H),
                                         int(V_shard), int(vocab_offset), int(V_total), int(chunk_size),
                                         float(temperature), partial or None, workspace or None,
                                         int(workspace_bytes), stream or None)


def raw_merge_shards(partials, P, targets, N, V_total, temperature, logp, entropy, lse, stream) -> int:
    """Call lmhead_logps_merge_shards with integer addresses (0 = NULL); returns the status."""
    return load().lmhead_logps_merge_shards(partials or None, int(P), targets or None, int(N), int(V_total),
                                            float(temperature), logp or None, entropy or None, lse or None,
                                            stream or None)


def raw_bwd_shard(hidden, W_shard, targets, N, H, V_shard, vocab_offset, V_total, chunk_size, temperature, lse,
                  entropy, g_logp, g_ent, dh, dW_shard, flags, workspace, workspace_bytes, stream) -> int:
    """Call lmhead_logps_bwd_shard with integer addresses (0 = NULL); returns the status."""
    return load().lmhead_logps_bwd_shard(hidden or None, W_shard or None, targets or None, int(N), int(H),
                                         int(V_shard), int(vocab_offset), int(V_total), int(chunk_size),
                                         float(temperature), lse or None, entropy or None, g_logp or None,
                                         g_ent or None, dh or None, dW_shard or None, int(flags),
                                         workspace or None, int(workspace_bytes), stream or None)


NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024


def raw_fwd_noalloc(hidden, W, targets, N, H, V, chunk_size, temperature, logp, entropy, lse, stream) -> int:
    """Call lmhead_logps_fwd_noalloc with integer addresses (0 = NULL); returns the status."""
    return load().lmhead_logps_fwd_noalloc(hidden or None, W or None, targets or None, int(N), int(H), int(V),
                                           int(chunk_size), float(temperature), logp or None, entropy or None,
                                           lse or None, stream or None)


TRACE_KERNELS = ("fwd_stats_kernel", "fwd_merge_kernel", "bwd_step_kernel", "transpose_kernel",
                 "fill_zero_kernel", "pad_rows_kernel", "bwd_step_bf16_kernel")


def trace_enable(on: bool) -> None:
    check(load().lmhead_logps_trace_enable(1 if on else 0))


def trace_read() -> dict:
    """{kernel name: {launches, ms, flops, bytes}} of the launches recorded
    since tracing was enabled (waits for them to finish)."""
    lib = load()
    out = {}
    for k in range(len(TRACE_KERNELS)):
        n = ctypes.c_int64(0)
        ms, fl, by = ctypes.c_double(0), ctypes.c_double(0), ctypes.c_double(0)
        check(lib.lmhead_logps_trace_read(k, ctypes.byref(n), ctypes.byref(ms), ctypes.byref(fl), ctypes.byref(by)))
        out[lib.lmhead_logps_trace_kernel_name(k).decode()] = {
            "launches": int(n.value), "ms": ms.value, "flops": fl.value, "bytes": by.value}
    return out


def version() -> str:
    return load().lmhead_logps_version().decode()
