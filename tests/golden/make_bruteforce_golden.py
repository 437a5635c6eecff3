"""Writes ``bruteforce_h64.json``: a small head case (N=4, H=64, V=19, one
masked token) whose forward values and gradients come from the 50-digit brute
force in ``oracle/bruteforce.py`` only. Inputs are drawn here with a fixed
seed and stored as bf16 bit patterns, so the file is self-contained.

Run from the repository root:  python tests/golden/make_bruteforce_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import bruteforce as B  # noqa: E402


def _bf16_bits(x):
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def main():
    rng = np.random.Generator(np.random.PCG64(20261202))
    N, H, V = 4, 64, 19
    h = _bf16_bits(rng.standard_normal((N, H)))
    W = _bf16_bits(rng.standard_normal((V, H)) * 0.25)
    t = rng.integers(0, V, size=N).astype(np.int64)
    t[2] = -1
    g_l = np.round(rng.standard_normal(N), 6)
    g_e = np.round(rng.standard_normal(N) * 0.5, 6)
    fwd = B.forward(h.tolist(), W.tolist(), t.tolist())
    dh, dW = B.gradients(h.tolist(), W.tolist(), t.tolist(), g_l, g_e)
    out = {
        "source": "oracle/bruteforce.py (50-digit decimal, unshifted definitions; "
                  "gradients by central differences at step 1e-20)",
        "N": N, "H": H, "V": V, "chunk_size": 3,
        "hidden_bf16_bits": h.tolist(),
        "W_bf16_bits": W.tolist(),
        "targets": t.tolist(),
        "g_logp": g_l.tolist(),
        "g_ent": g_e.tolist(),
        "logp": [str(x[0]) for x in fwd],
        "entropy": [str(x[1]) for x in fwd],
        "lse": [str(x[2]) for x in fwd],
        "dh": [[str(v) for v in row] for row in dh],
        "dW": [[str(v) for v in row] for row in dW],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "bruteforce_h64.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
