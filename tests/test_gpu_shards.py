"""The head over vocabulary shards on the GPU (tunix #2913 runs its head with
the vocabulary table split across devices and combines the per-token partials
across shards; here the shards run one after another on one GPU): per-shard
partial records merged by log-sum-exp, and per-shard backward with dh added
across shards, against the fp64 oracle of the whole vocabulary and against the
whole-table GPU path. Includes the pages' 248,320-entry vocabulary."""
import numpy as np
import pytest

import oracle.lmhead_oracle as O
from gpu_common import assert_grad_close, assert_stats_close, dev, dev_bits, log, run_head
from synthetic import f32_to_bf16_bits, sample_tokens

pytestmark = pytest.mark.gpu


def _case(seed, N, H, V, w_std=0.05, n_masked=0, rms_one=False):
    rng = np.random.default_rng(seed)
    hf = rng.standard_normal((N, H)).astype(np.float32)
    if rms_one:
        hf /= np.sqrt(np.mean(hf * hf, axis=1, keepdims=True))
    h = f32_to_bf16_bits(hf)
    W = f32_to_bf16_bits((rng.standard_normal((V, H)) * w_std).astype(np.float32))
    t = rng.integers(0, V, size=N).astype(np.int32)
    if n_masked:
        t[rng.choice(N, size=n_masked, replace=False)] = -1
    g_l = rng.standard_normal(N).astype(np.float32)
    g_e = (rng.standard_normal(N) * 0.1).astype(np.float32)
    return h, W, t, g_l, g_e


def run_sharded(h, W, t, C, bounds, g_l=None, g_e=None, T=1.0, backward=True):
    """Forward over the shards [bounds[p], bounds[p+1]), merge, then the
    per-shard backward (dh added across shards); numpy outputs."""
    import torch
    import cross_entropy_amd as lm
    from cross_entropy_amd import _native as nat
    N, H = h.shape
    V = W.shape[0]
    P = len(bounds) - 1
    hd, td = dev_bits(h), dev(t)
    shards = [dev_bits(np.ascontiguousarray(W[bounds[p]:bounds[p + 1]])) for p in range(P)]
    parts = torch.empty((P, N, 4), dtype=torch.float32, device="cuda")
    for p in range(P):
        ws = lm.workspace_for(hd, shards[p], C, with_backward=False)
        lm.lmhead_logps_fwd_shard(hd, shards[p], td, bounds[p], V, C, T, parts[p], ws)
    logp = torch.empty(N, device="cuda")
    ent = torch.empty(N, device="cuda")
    lse = torch.empty(N, device="cuda")
    lm.lmhead_logps_merge_shards(parts, td, V, T, logp, ent, lse)
    out = {"logp": logp, "entropy": ent, "lse": lse}
    if backward:
        gl, ge = dev(g_l), dev(g_e)
        dh = torch.empty((N, H), device="cuda")
        dWs = []
        for p in range(P):
            ws = lm.workspace_for(hd, shards[p], C, with_backward=True)
            dWp = torch.empty((bounds[p + 1] - bounds[p], H), device="cuda")
            flags = 0 if p == 0 else nat.BWD_ACCUMULATE_DH
            lm.lmhead_logps_bwd_shard(hd, shards[p], td, bounds[p], V, C, T, lse, ent, gl, ge, dh, dWp, flags, ws)
            dWs.append(dWp)
        out["dh"] = dh
        out["dW"] = torch.cat(dWs, dim=0)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


@pytest.mark.parametrize("T", [1.0, 0.7])
@pytest.mark.parametrize("bounds", [[0, 1700, 3748, 5000], [0, 1000, 2000, 3000, 4000, 5000], [0, 5000]])
def test_sharded_head_matches_oracle(bounds, T):
    h, W, t, g_l, g_e = _case(51, 700, 256, 5000, n_masked=20)
    log(f"[shards] bounds {bounds} T={T}")
    got = run_sharded(h, W, t, 96, bounds, g_l, g_e, T=T)
    ref = O.forward_backward(h, W, t, 96, g_l, g_e, temperature=T)
    valid = t >= 0
    for k in ("logp", "entropy", "lse"):
        assert_stats_close(got[k][valid], ref[k][valid], f"shards {k}")
        assert np.all(got[k][~valid] == 0.0)
    assert np.all(got["dh"][~valid] == 0.0)
    assert_grad_close(got["dh"], ref["dh"], "shards dh")
    assert_grad_close(got["dW"], ref["dW"], "shards dW")


def test_random_shard_splits():
    """A seeded sweep: random shapes, 1 to 6 shards cut at random rows (a
    shard may be a single row), temperatures 0.7 to 1.3, masked ids -1 and
    V; the merged statistics and the per-shard gradients against the oracle
    of the whole vocabulary."""
    rng = np.random.default_rng(4711)
    for case in range(8):
        N = int(rng.integers(1, 900))
        H = 64 * int(rng.integers(1, 6))
        V = int(rng.integers(8, 5000))
        C = int(rng.integers(1, N + 50))
        P = int(rng.integers(1, 7))
        cuts = sorted(set(int(x) for x in rng.integers(1, V, size=P - 1)))
        if case == 0:
            cuts = sorted(set(cuts + [1, V - 1]))   # one-row shards at both ends
        bounds = [0] + cuts + [V]
        T = (1.0, 0.7, 1.3)[case % 3]
        h, W, t, g_l, g_e = _case(600 + case, N, H, V, w_std=float(rng.uniform(0.02, 0.2)),
                                  n_masked=int(rng.integers(0, N // 4 + 1)))
        if N > 1:
            t[int(rng.integers(0, N))] = V      # out of the whole vocabulary: masked
        what = f"random shards {case}: N={N} H={H} V={V} C={C} bounds={bounds} T={T}"
        log(f"[shards] {what}")
        got = run_sharded(h, W, t, C, bounds, g_l, g_e, T=T)
        ref = O.forward_backward(h, W, t, C, g_l, g_e, temperature=T)
        valid = (t >= 0) & (t < V)
        for k in ("logp", "entropy", "lse"):
            assert_stats_close(got[k][valid], ref[k][valid], f"{what} {k}")
            assert np.all(got[k][~valid] == 0.0), f"{what} masked {k}"
        assert np.all(got["dh"][~valid] == 0.0), f"{what} masked dh"
        assert_grad_close(got["dh"], ref["dh"], f"{what} dh")
        assert_grad_close(got["dW"], ref["dW"], f"{what} dW")


def test_one_shard_is_the_whole_table_bit_for_bit():
    """One shard covering the vocabulary, merged alone, gives the plain
    forward's bits (the same split records and merge arithmetic)."""
    h, W, t, g_l, g_e = _case(52, 513, 128, 4097, n_masked=9)
    a = run_sharded(h, W, t, 64, [0, 4097], g_l, g_e)
    b = run_head(h, W, t, 64, g_l, g_e)
    for k in ("logp", "entropy", "lse", "dh", "dW"):
        assert np.array_equal(a[k], b[k]), k


def test_pages_vocabulary_248320_sharded_and_whole():
    """The pages' 248,320-entry vocabulary (Qwen3.5-397B-A17B's; the pages give
    no hidden size, 2,560 is used), 4,096 tokens: the whole-table path and a
    4-way shard split against the oracle on sampled tokens; dW on a run with
    cotangents zeroed outside the sample."""
    N, H, V, C = 4096, 2560, 248320, 512
    h, W, t, g_l, g_e = _case(53, N, H, V, w_std=0.02, rms_one=True)
    idx = sample_tokens(t, 48, seed=53)
    sl, se = np.zeros_like(g_l), np.zeros_like(g_e)
    sl[idx], se[idx] = g_l[idx], g_e[idx]
    log("[shards] V=248320: oracle on the sample")
    ref_lp, ref_en, ref_lse = O.forward(h, W, t, C, tokens=idx)
    ref_dh, ref_dW = O.backward(h, W, t, C, sl, se, tokens=idx)
    bounds = [0, 62080, 124160, 186240, 248320]
    for name, got in (("whole", None), ("4 shards", None)):
        log(f"[shards] V=248320 {name}: GPU")
        if name == "whole":
            got = run_head(h, W, t, C, sl, se)
        else:
            got = run_sharded(h, W, t, C, bounds, sl, se)
        for k, ref in (("logp", ref_lp), ("entropy", ref_en), ("lse", ref_lse)):
            assert_stats_close(got[k][idx], ref, f"V=248320 {name} {k}")
        assert_grad_close(got["dh"][idx], ref_dh, f"V=248320 {name} dh (sampled rows)")
        assert_grad_close(got["dW"], ref_dW, f"V=248320 {name} dW (sparse cotangents)")
