"""HIP path vs the fp64 oracle, through the C ABI, on seeded inputs.

Small shapes are compared element by element in full (several tiles, ragged
tails in every dimension, many backward blocks). The five workloads run at
their full sizes in the launch configuration the benchmark times; there the
oracle evaluates a fixed sample of tokens one by one (each token needs only
its own logits row), and dW is checked on the same inputs with cotangents
zeroed outside that sample, which the oracle then evaluates exactly."""
import json
import os

import numpy as np
import pytest

import oracle.lmhead_oracle as O
from gpu_common import assert_grad_close, assert_stats_close, log, run_head
from synthetic import WORKLOADS, make_cotangents, make_inputs, sample_tokens

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand_bits(rng, shape, std):
    from synthetic import f32_to_bf16_bits
    return f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(std))


def _case(seed, N, H, V, w_std=0.05, n_masked=0, masked_ids=(-1,)):
    rng = np.random.default_rng(seed)
    h = _rand_bits(rng, (N, H), 1.0)
    W = _rand_bits(rng, (V, H), w_std)
    t = rng.integers(0, V, size=N).astype(np.int32)
    if n_masked:
        idx = rng.choice(N, size=n_masked, replace=False)
        t[idx] = np.resize(np.array(masked_ids, dtype=np.int32), n_masked)
    g_l = rng.standard_normal(N).astype(np.float32)
    g_e = (rng.standard_normal(N) * 0.1).astype(np.float32)
    return h, W, t, g_l, g_e


def _check_full(h, W, t, C, g_l, g_e, what):
    log(f"[parity] {what}: N={h.shape[0]} H={h.shape[1]} V={W.shape[0]} C={C}")
    got = run_head(h, W, t, C, g_l, g_e)
    ref = O.forward_backward(h, W, t, C, g_l, g_e)
    V = W.shape[0]
    valid = (t >= 0) & (t < V)
    for k in ("logp", "entropy", "lse"):
        assert_stats_close(got[k][valid], ref[k][valid], f"{what} {k}")
        assert np.all(got[k][~valid] == 0.0), f"{what} masked {k}"
    assert np.all(got["dh"][~valid] == 0.0), f"{what} masked dh rows"
    rh = assert_grad_close(got["dh"], ref["dh"], f"{what} dh")
    rw = assert_grad_close(got["dW"], ref["dW"], f"{what} dW")
    log(f"[parity] {what}: dh frob {rh:.2e}, dW frob {rw:.2e}")
    return got


def test_golden_bruteforce_case():
    """GPU vs the stored 50-digit brute-force values (one partial tile in
    every dimension, one masked token)."""
    g = json.load(open(os.path.join(GOLDEN, "bruteforce_h64.json")))
    h = np.array(g["hidden_bf16_bits"], dtype=np.uint16)
    W = np.array(g["W_bf16_bits"], dtype=np.uint16)
    t = np.array(g["targets"], dtype=np.int32)
    log("[parity] golden brute-force case")
    got = run_head(h, W, t, g["chunk_size"], np.array(g["g_logp"], np.float32), np.array(g["g_ent"], np.float32))
    valid = t >= 0
    for k in ("logp", "entropy", "lse"):
        ref = np.array([float(x) for x in g[k]])
        assert_stats_close(got[k][valid], ref[valid], f"golden {k}")
        assert np.all(got[k][~valid] == 0.0)
    for k in ("dh", "dW"):
        ref = np.array([[float(x) for x in row] for row in g[k]])
        assert_grad_close(got[k], ref, f"golden {k}")


@pytest.mark.parametrize("N,H,V,C,n_masked", [
    (256, 256, 4096, 128, 0),      # the tiny workload's sizes, own seed
    (300, 128, 1000, 64, 17),      # ragged tokens and vocabulary
    (700, 320, 3001, 7, 40),       # H not a multiple of 256; tiny chunk -> 3 x 12 backward blocks
    (513, 256, 4097, 4096, 5),     # one chunk larger than N; vocabulary one past a tile
    (64, 64, 5, 1, 3),             # fewer vocabulary rows than one MFMA block
    (2048, 256, 20000, 512, 9),    # 27 forward splits of 3 chained vocabulary tiles; the last tile ragged
    (1, 128, 777, 1, 0),           # one token: one cotangent tile per launch, 7 XCDs with nothing to take
])
def test_parity_full_small(N, H, V, C, n_masked):
    h, W, t, g_l, g_e = _case(N * 7 + V, N, H, V, n_masked=n_masked, masked_ids=(-1, V, -3))
    _check_full(h, W, t, C, g_l, g_e, f"small({N},{H},{V},{C})")


def test_parity_tiny_workload_full():
    """Workload 1 exactly as specified, full comparison."""
    cfg = WORKLOADS[1]
    h, W, t = make_inputs(cfg)
    g_l, g_e = make_cotangents(cfg)
    _check_full(h, W, t, cfg.chunk_size, g_l, g_e, "workload 1")


@pytest.mark.parametrize("workload_no,chunk", [(2, 512), (3, 512), (4, 1024), (4, 4096), (5, 4096)])
def test_parity_workload_sampled(workload_no, chunk):
    """Full-size workloads: all outputs computed on the GPU, the oracle
    evaluates 128 sampled tokens (plus masked samples) one by one; dW is
    checked on a second backward whose cotangents vanish outside the sample."""
    cfg = WORKLOADS[workload_no]
    log(f"[parity] workload {workload_no} chunk {chunk}: generating inputs")
    h, W, t = make_inputs(cfg)
    g_l, g_e = make_cotangents(cfg)
    V = cfg.V
    log(f"[parity] workload {workload_no}: GPU dense run")
    got = run_head(h, W, t, chunk, g_l, g_e)
    valid = (t >= 0) & (t < V)
    for k in ("logp", "entropy", "lse"):
        assert np.all(got[k][~valid] == 0.0), f"masked {k}"
        assert np.all(np.isfinite(got[k])), f"non-finite {k}"
    assert np.all(got["dh"][~valid] == 0.0), "masked dh rows"
    idx = sample_tokens(t, 128, seed=workload_no, include_masked=8)
    log(f"[parity] workload {workload_no}: oracle on {idx.size} sampled tokens")
    ref_lp, ref_en, ref_lse = O.forward(h, W, t, chunk, tokens=idx)
    for k, ref in (("logp", ref_lp), ("entropy", ref_en), ("lse", ref_lse)):
        assert_stats_close(got[k][idx], ref, f"workload {workload_no} {k}")
    sl = np.zeros_like(g_l)
    se = np.zeros_like(g_e)
    sl[idx], se[idx] = g_l[idx], g_e[idx]
    ref_dh, ref_dW = O.backward(h, W, t, chunk, sl, se, tokens=idx)
    rh = assert_grad_close(got["dh"][idx], ref_dh, f"workload {workload_no} dh (sampled rows)")
    log(f"[parity] workload {workload_no}: GPU sparse-cotangent run")
    sparse = run_head(h, W, t, chunk, sl, se)
    rw = assert_grad_close(sparse["dW"], ref_dW, f"workload {workload_no} dW (sparse cotangents)")
    assert np.array_equal(sparse["dh"][idx], got["dh"][idx]), "dh rows depend only on their own cotangents"
    log(f"[parity] workload {workload_no}: dh frob {rh:.2e}, dW frob {rw:.2e}")
