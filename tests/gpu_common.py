"""Helpers shared by the GPU tests: device copies of seeded inputs, one call
of the HIP path through the C ABI, and the comparison bar.

Bar (stated for this head): logp, entropy and lse within
|gpu - oracle| <= 2e-3 + 1e-3 |oracle| per unmasked token; dh and dW within
5e-3 relative Frobenius error; masked tokens exactly 0."""
from __future__ import annotations

import sys

import numpy as np

ATOL, RTOL, FROB = 2e-3, 1e-3, 5e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bits(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")


def dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def run_head(h_bits, W_bits, targets, chunk_size, g_l=None, g_e=None, with_entropy=True, backward=True,
             entropy_grad=True, temperature=None):
    """Forward (and backward) on the GPU; returns numpy arrays. ``temperature``
    None runs the plain entry points, a number the tempered ones."""
    import torch
    import cross_entropy_amd as lm
    h, W, t = dev_bits(h_bits), dev_bits(W_bits), dev(targets.astype(np.int32))
    ws = lm.workspace_for(h, W, chunk_size, with_backward=True)
    logp, ent, lse = lm.forward(h, W, t, chunk_size, with_entropy=with_entropy, workspace=ws,
                                temperature=temperature)
    out = {"logp": logp, "entropy": ent, "lse": lse}
    if backward:
        gl = None if g_l is None else dev(np.asarray(g_l, dtype=np.float32))
        ge = None if (g_e is None or not entropy_grad) else dev(np.asarray(g_e, dtype=np.float32))
        dh, dW = lm.backward(h, W, t, chunk_size, lse, ent if ge is not None else None, gl, ge, workspace=ws,
                             temperature=temperature)
        out["dh"], out["dW"] = dh, dW
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu().numpy()) for k, v in out.items()}


def assert_stats_close(gpu, ref, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(gpu - ref)
    lim = ATOL + RTOL * np.abs(ref)
    bad = np.flatnonzero(~(err <= lim))
    assert bad.size == 0, (f"{what}: {bad.size} tokens out of tolerance, worst at {bad[np.argmax(err[bad])]}: "
                           f"gpu {gpu[bad[0]]!r} oracle {ref[bad[0]]!r}")


def frob_rel(gpu, ref) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    n = np.linalg.norm(ref)
    d = np.linalg.norm(gpu - ref)
    if n == 0.0:
        return 0.0 if d == 0.0 else float("inf")
    return float(d / n)


def assert_grad_close(gpu, ref, what=""):
    r = frob_rel(gpu, ref)
    assert r <= FROB, f"{what}: relative Frobenius error {r:.3e} > {FROB}"
    return r
