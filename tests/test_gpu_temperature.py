"""The tempered head on the GPU (logits divided by T; google/tunix pull
request #2913 runs its head at temperatures 1 and 0.7) against the fp64
oracle at the same temperature, through the C ABI's tempered entry points."""
import numpy as np
import pytest

import oracle.lmhead_oracle as O
from gpu_common import assert_grad_close, assert_stats_close, log, run_head
from synthetic import WORKLOADS, f32_to_bf16_bits, make_cotangents, make_inputs, sample_tokens

pytestmark = pytest.mark.gpu


def _case(seed, N, H, V, w_std=0.05, n_masked=0):
    rng = np.random.default_rng(seed)
    h = f32_to_bf16_bits(rng.standard_normal((N, H)).astype(np.float32))
    W = f32_to_bf16_bits((rng.standard_normal((V, H)) * w_std).astype(np.float32))
    t = rng.integers(0, V, size=N).astype(np.int32)
    if n_masked:
        t[rng.choice(N, size=n_masked, replace=False)] = -1
    g_l = rng.standard_normal(N).astype(np.float32)
    g_e = (rng.standard_normal(N) * 0.1).astype(np.float32)
    return h, W, t, g_l, g_e


@pytest.mark.parametrize("T", [0.7, 2.0, 0.25])
@pytest.mark.parametrize("N,H,V,C,n_masked", [(300, 128, 1000, 64, 17), (513, 256, 4097, 96, 5)])
def test_tempered_parity_full_small(T, N, H, V, C, n_masked):
    h, W, t, g_l, g_e = _case(N + V + int(100 * T), N, H, V, n_masked=n_masked)
    log(f"[temperature] T={T} N={N} H={H} V={V} C={C}")
    got = run_head(h, W, t, C, g_l, g_e, temperature=T)
    ref = O.forward_backward(h, W, t, C, g_l, g_e, temperature=T)
    valid = (t >= 0) & (t < V)
    for k in ("logp", "entropy", "lse"):
        assert_stats_close(got[k][valid], ref[k][valid], f"T={T} {k}")
        assert np.all(got[k][~valid] == 0.0), f"T={T} masked {k}"
    assert np.all(got["dh"][~valid] == 0.0)
    assert_grad_close(got["dh"], ref["dh"], f"T={T} dh")
    assert_grad_close(got["dW"], ref["dW"], f"T={T} dW")


def test_temperature_one_is_the_plain_head_bit_for_bit():
    h, W, t, g_l, g_e = _case(7, 300, 128, 1000, n_masked=9)
    a = run_head(h, W, t, 64, g_l, g_e)
    b = run_head(h, W, t, 64, g_l, g_e, temperature=1.0)
    for k in ("logp", "entropy", "lse", "dh", "dW"):
        assert np.array_equal(a[k], b[k]), k


def test_power_of_two_temperature_equals_scaled_W():
    """T = 2 scores what T = 1 scores with W halved (exact in bf16): the GPU's
    statistics and dh agree to float32 rounding, and dW(T=2) = dW(W/2) / 2."""
    h, W, t, g_l, g_e = _case(8, 256, 128, 2048)
    W_half = f32_to_bf16_bits((O.widen_bf16(W) * 0.5).astype(np.float32))
    a = run_head(h, W, t, 64, g_l, g_e, temperature=2.0)
    b = run_head(h, W_half, t, 64, g_l, g_e)
    for k in ("logp", "entropy", "lse"):
        assert_stats_close(a[k], b[k], f"T=2 vs W/2 {k}")
    assert_grad_close(a["dh"], b["dh"], "T=2 vs W/2 dh")
    assert_grad_close(a["dW"], 0.5 * b["dW"], "T=2 vs W/2 dW")


def test_tempered_workload_2_sampled():
    """The one-sequence Qwen3-4B-shaped head (N 4096, H 2560, V 151936,
    chunk 512) at T = 0.7: sampled tokens against the oracle; dW on a second
    run with cotangents zeroed outside the sample."""
    cfg = WORKLOADS[2]
    h, W, t = make_inputs(cfg)
    g_l, g_e = make_cotangents(cfg)
    T = 0.7
    log("[temperature] workload 2 at T=0.7: GPU dense run")
    got = run_head(h, W, t, cfg.chunk_size, g_l, g_e, temperature=T)
    idx = sample_tokens(t, 96, seed=72)
    ref_lp, ref_en, ref_lse = O.forward(h, W, t, cfg.chunk_size, tokens=idx, temperature=T)
    for k, ref in (("logp", ref_lp), ("entropy", ref_en), ("lse", ref_lse)):
        assert_stats_close(got[k][idx], ref, f"workload 2 T=0.7 {k}")
    sl, se = np.zeros_like(g_l), np.zeros_like(g_e)
    sl[idx], se[idx] = g_l[idx], g_e[idx]
    ref_dh, ref_dW = O.backward(h, W, t, cfg.chunk_size, sl, se, tokens=idx, temperature=T)
    assert_grad_close(got["dh"][idx], ref_dh, "workload 2 T=0.7 dh (sampled rows)")
    log("[temperature] workload 2 at T=0.7: GPU sparse-cotangent run")
    sparse = run_head(h, W, t, cfg.chunk_size, sl, se, temperature=T)
    assert_grad_close(sparse["dW"], ref_dW, "workload 2 T=0.7 dW (sparse cotangents)")
