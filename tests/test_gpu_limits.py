"""Sizes at the library's limits, through the C ABI, against the oracle on
sampled tokens: a hidden tensor of more than 2^31 elements (every address
in the kernels is 64-bit where a product of a token index and H can pass
2^31), and a vocabulary at the backward's bound (V rounded up to 256 stays
below 2^23), ragged."""
import numpy as np
import pytest

import oracle.lmhead_oracle as O
from gpu_common import assert_grad_close, assert_stats_close, log
from synthetic import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _normal_bits(rng, shape, std, rows=1 << 16):
    out = np.empty(shape, dtype=np.uint16)
    for r0 in range(0, shape[0], rows):
        r1 = min(shape[0], r0 + rows)
        out[r0:r1] = f32_to_bf16_bits(rng.standard_normal((r1 - r0,) + tuple(shape[1:]), dtype=np.float32)
                                      * np.float32(std))
    return out


def _run_sampled(h, W, t, C, g_l, g_e, idx, what):
    import torch
    import cross_entropy_amd as lm
    from gpu_common import dev, dev_bits
    hd, Wd, td = dev_bits(h), dev_bits(W), dev(t)
    sl = np.zeros_like(g_l)
    se = np.zeros_like(g_e)
    sl[idx], se[idx] = g_l[idx], g_e[idx]
    ws = lm.workspace_for(hd, Wd, C, with_backward=True)
    logp, ent, lse = lm.forward(hd, Wd, td, C, workspace=ws)
    dh, dW = lm.backward(hd, Wd, td, C, lse, ent, dev(sl), dev(se), workspace=ws)
    torch.cuda.synchronize()
    got = {"logp": logp.cpu().numpy(), "entropy": ent.cpu().numpy(), "lse": lse.cpu().numpy(),
           "dh": dh[torch.from_numpy(idx).cuda()].cpu().numpy(), "dW": dW.cpu().numpy()}
    del hd, Wd, ws, dh, dW
    torch.cuda.empty_cache()
    log(f"[limits] {what}: oracle on {idx.size} tokens")
    ref_lp, ref_en, ref_lse = O.forward(h, W, t, C, tokens=idx)
    valid = (t[idx] >= 0) & (t[idx] < W.shape[0])
    for k, r in (("logp", ref_lp), ("entropy", ref_en), ("lse", ref_lse)):
        assert_stats_close(got[k][idx][valid], r[valid], f"{what} {k}")
        assert np.all(got[k][idx][~valid] == 0.0)
    ref_dh, ref_dW = O.backward(h, W, t, C, sl, se, tokens=idx)
    rh = assert_grad_close(got["dh"], ref_dh, f"{what} dh (sampled rows)")
    rw = assert_grad_close(got["dW"], ref_dW, f"{what} dW (sampled cotangents)")
    log(f"[limits] {what}: dh frob {rh:.2e}, dW frob {rw:.2e}")


@pytest.mark.timeout(600)
def test_hidden_beyond_2_to_31_elements():
    N, H, V, C = 2_200_000, 1024, 512, 4096     # N * H = 2.25e9 > 2^31
    rng = np.random.default_rng(2024)
    log(f"[limits] generating hidden [{N}, {H}] (4.5 GB)")
    h = _normal_bits(rng, (N, H), 1.0)
    W = _normal_bits(rng, (V, H), 0.03)
    t = rng.integers(0, V, size=N).astype(np.int32)
    t[rng.choice(N, size=1000, replace=False)] = -1
    g_l = rng.standard_normal(N).astype(np.float32)
    g_e = (rng.standard_normal(N) * 0.1).astype(np.float32)
    # the sample reaches the last tokens, whose hidden rows lie past 2^31 elements
    idx = np.unique(np.concatenate([rng.choice(N, 380, replace=False), np.arange(N - 100, N),
                                    np.flatnonzero(t < 0)[:20], [0, 2_097_151, 2_097_152]])).astype(np.int64)
    _run_sampled(h, W, t, C, g_l, g_e, idx, "N = 2.2M, H = 1024")


@pytest.mark.timeout(600)
def test_vocabulary_at_the_backward_bound():
    V = (1 << 23) - 256 - 5                       # rounded up to 256: 2^23 - 256
    N, H, C = 700, 64, 64
    rng = np.random.default_rng(2025)
    log(f"[limits] vocabulary of {V}")
    h = _normal_bits(rng, (N, H), 1.0)
    W = _normal_bits(rng, (V, H), 0.2)
    t = rng.integers(0, V, size=N).astype(np.int32)
    t[:3] = [V - 1, 0, V - 257]
    t[rng.choice(np.arange(3, N), size=9, replace=False)] = -1
    g_l = rng.standard_normal(N).astype(np.float32)
    g_e = (rng.standard_normal(N) * 0.1).astype(np.float32)
    idx = np.unique(np.concatenate([[0, 1, 2], rng.choice(N, 45, replace=False)])).astype(np.int64)
    _run_sampled(h, W, t, C, g_l, g_e, idx, f"V = {V}")
