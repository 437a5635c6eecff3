"""The C ABI from a C++ caller with no Python and no PyTorch
(tests/capi/capi_check.cpp, built with the library and linked against the
system HIP runtime): it allocates with hipMalloc, runs the forward and the
backward on a stream of its own, and writes its outputs, which must meet the
oracle's bar and equal, bit for bit, the outputs of the same calls made
through the Python binding."""
import os
import subprocess

import numpy as np
import pytest

import oracle.lmhead_oracle as O
from gpu_common import assert_grad_close, assert_stats_close, log, run_head
from synthetic import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "capi", "capi_check")


def test_c_caller_without_python(tmp_path):
    assert os.path.exists(BIN), f"{BIN} is missing: run __graft_entry__.build()"
    N, H, V, C = 1500, 256, 5003, 96
    rng = np.random.default_rng(99)
    h = f32_to_bf16_bits(rng.standard_normal((N, H)).astype(np.float32))
    W = f32_to_bf16_bits((rng.standard_normal((V, H)) * 0.05).astype(np.float32))
    t = rng.integers(0, V, size=N).astype(np.int32)
    t[rng.choice(N, size=25, replace=False)] = -1
    g_l = rng.standard_normal(N).astype(np.float32)
    g_e = (rng.standard_normal(N) * 0.1).astype(np.float32)
    d = str(tmp_path)
    with open(os.path.join(d, "dims.txt"), "w") as f:
        f.write(f"{N} {H} {V} {C}\n")
    for name, a in (("hidden", h), ("W", W), ("targets", t), ("g_logp", g_l), ("g_ent", g_e)):
        np.ascontiguousarray(a).tofile(os.path.join(d, name + ".bin"))
    log("[capi] running the C++ caller")
    r = subprocess.run([BIN, d], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-2000:])
    assert "capi_check: ok" in r.stdout
    got = {k: np.fromfile(os.path.join(d, k + ".bin"), dtype=np.float32)
           for k in ("logp", "entropy", "lse", "dh", "dW")}
    got["dh"] = got["dh"].reshape(N, H)
    got["dW"] = got["dW"].reshape(V, H)
    ref = O.forward_backward(h, W, t, C, g_l, g_e)
    valid = t >= 0
    for k in ("logp", "entropy", "lse"):
        assert_stats_close(got[k][valid], ref[k][valid], f"C caller {k}")
        assert np.all(got[k][~valid] == 0.0)
    assert_grad_close(got["dh"], ref["dh"], "C caller dh")
    assert_grad_close(got["dW"], ref["dW"], "C caller dW")
    py = run_head(h, W, t, C, g_l, g_e)
    for k in ("logp", "entropy", "lse", "dh", "dW"):
        assert np.array_equal(got[k].view(np.uint32), np.ascontiguousarray(py[k]).view(np.uint32)), \
            f"{k}: the C caller and the Python binding differ"
