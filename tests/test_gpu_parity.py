"""HIP path vs the fp64 oracle, through the C ABI, on seeded inputs.

Small shapes are compared element by element in full (several tiles, ragged
tails in every dimension, many backward blocks). The one-sequence workload
(N 4096, H 2560, V 151936) is compared in full: every token's statistics,
all of dh and all of dW under the real dense cotangents. The other workloads
run at their full sizes in the launch configuration the benchmark times;
there the oracle evaluates a fixed sample of 1,024 tokens one by one (each
token needs only its own logits row), and dW is checked on the same inputs
with cotangents zeroed outside that sample, which the oracle then evaluates
exactly. Peaked logits (logit std 8 to 16, targets planted at +30 so their
probability rounds to 1, a row of logits near +80) cover the numerical edges
of a trained head: the cancellation in onehot - p, the base-2 running-max
rescale at large logits and near-zero entropy."""
import json
import os

import numpy as np
import pytest

import oracle.lmhead_oracle as O
from gpu_common import assert_grad_close, assert_stats_close, log, run_head
from synthetic import WORKLOADS, f32_to_bf16_bits, make_cotangents, make_inputs, sample_tokens

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
    (129, 192, 2, 16, 4),          # two vocabulary rows
])
def test_parity_full_small(N, H, V, C, n_masked):
    h, W, t, g_l, g_e = _case(N * 7 + V, N, H, V, n_masked=n_masked, masked_ids=(-1, V, -3))
    _check_full(h, W, t, C, g_l, g_e, f"small({N},{H},{V},{C})")


def test_parity_one_vocabulary_row():
    """V = 1: p = 1 for every token, so logp = entropy = 0, lse = z and both
    gradients are exactly 0 in the oracle. The head's float32 arithmetic forms
    log2 p as the difference of z log2(e) and lse log2(e), each rounded, so its
    p is 1 only up to a few ulps of |z| and dz = g (1 - p) - g_ent p log p is
    rounding noise. The relative Frobenius bar is undefined against an exact
    zero; the gradients are instead bounded elementwise by that noise,
    |dz_i| <= (|g_l,i| + |g_ent,i|) 2^-20 (1 + |z_i|), carried through the two
    products."""
    N, H, V, C = 37, 64, 1, 8
    h, W, t, g_l, g_e = _case(4242, N, H, V, w_std=0.5, n_masked=2, masked_ids=(-1, 1))
    log(f"[parity] one vocabulary row: N={N} H={H} C={C}")
    got = run_head(h, W, t, C, g_l, g_e)
    ref = O.forward_backward(h, W, t, C, g_l, g_e)
    valid = (t >= 0) & (t < V)
    assert np.all(ref["dh"] == 0.0) and np.all(ref["dW"] == 0.0)
    for k in ("logp", "entropy", "lse"):
        assert_stats_close(got[k][valid], ref[k][valid], f"V=1 {k}")
        assert np.all(got[k][~valid] == 0.0), f"V=1 masked {k}"
    hf = O.widen_bf16(h)
    Wf = O.widen_bf16(W)
    z = hf @ Wf[0]
    dz_bound = np.where(valid, (np.abs(g_l) + np.abs(g_e)) * 2.0 ** -20 * (1.0 + np.abs(z)), 0.0)
    dh_bound = dz_bound[:, None] * np.abs(Wf[0])[None, :]
    dW_bound = dz_bound @ np.abs(hf)
    assert np.all(got["dh"][~valid] == 0.0), "V=1 masked dh rows"
    assert np.all(np.abs(got["dh"]) <= dh_bound), f"V=1 dh: max {np.abs(got['dh']).max():.3e}"
    assert np.all(np.abs(got["dW"][0]) <= dW_bound), f"V=1 dW: max {np.abs(got['dW']).max():.3e}"


def test_parity_random_shapes():
    """A seeded sweep of shapes the fixed cases do not pick: tokens 1 to
    1,200, H from 64 to 448 in steps of 64 (partial last H tiles), vocabulary
    2 to 6,000 (ragged last tiles and W tails), chunk sizes from 1 to past N,
    up to a third of the tokens masked (ids -1, V, -7), temperatures 0.7 to
    1.3, with and without the entropy cotangent; every output against the
    oracle."""
    rng = np.random.default_rng(31337)
    for case in range(16):
        N = int(rng.integers(1, 1201))
        H = 64 * int(rng.integers(1, 8))
        V = int(rng.integers(2, 6001))
        C = int(rng.integers(1, N + 101))
        T = (1.0, 0.7, 1.3)[case % 3]
        with_ent = case % 4 != 3
        n_masked = int(rng.integers(0, N // 3 + 1))
        h, W, t, g_l, g_e = _case(1000 + case, N, H, V, w_std=float(rng.uniform(0.02, 0.3)),
                                  n_masked=n_masked, masked_ids=(-1, V, -7))
        what = f"random {case}: N={N} H={H} V={V} C={C} T={T} entropy cotangent {with_ent}"
        log(f"[parity] {what}")
        got = run_head(h, W, t, C, g_l, g_e, entropy_grad=with_ent, temperature=T)
        ref = O.forward_backward(h, W, t, C, g_l, g_e if with_ent else None, temperature=T)
        valid = (t >= 0) & (t < V)
        for k in ("logp", "entropy", "lse"):
            assert_stats_close(got[k][valid], ref[k][valid], f"{what} {k}")
            assert np.all(got[k][~valid] == 0.0), f"{what} masked {k}"
        assert np.all(got["dh"][~valid] == 0.0), f"{what} masked dh rows"
        assert_grad_close(got["dh"], ref["dh"], f"{what} dh")
        assert_grad_close(got["dW"], ref["dW"], f"{what} dW")


def test_parity_tiny_workload_full():
    """Workload 1 exactly as specified, full comparison."""
    cfg = WORKLOADS[1]
    h, W, t = make_inputs(cfg)
    g_l, g_e = make_cotangents(cfg)
    _check_full(h, W, t, cfg.chunk_size, g_l, g_e, "workload 1")


@pytest.mark.timeout(900)
def test_parity_workload2_full():
    """The one-sequence workload compared in full: every token's logp,
    entropy and lse, all of dh, and all of dW under the dense cotangents."""
    cfg = WORKLOADS[2]
    h, W, t = make_inputs(cfg)
    g_l, g_e = make_cotangents(cfg)
    _check_full(h, W, t, cfg.chunk_size, g_l, g_e, "workload 2 (full)")


@pytest.mark.slow
@pytest.mark.timeout(3000)
@pytest.mark.parametrize("chunk", [1024])
def test_parity_workload4_full(chunk):
    """The context-rank share (N 15237, H 4096) compared in full; about 10
    minutes of host BLAS, so it runs only with --run-slow."""
    cfg = WORKLOADS[4]
    h, W, t = make_inputs(cfg)
    g_l, g_e = make_cotangents(cfg)
    what = f"workload 4 chunk {chunk} (full)"
    log(f"[parity] {what}: GPU run")
    got = run_head(h, W, t, chunk, g_l, g_e)
    N, V = t.size, cfg.V
    valid = (t >= 0) & (t < V)
    # the oracle over disjoint token ranges (each range's dW sums only its own
    # tokens; the ranges' sum is the full dW), logging as it goes
    ref_dW = np.zeros((V, cfg.H))
    step = 2048
    for a in range(0, N, step):
        idx = np.arange(a, min(N, a + step))
        lp, en, ls = O.forward(h, W, t, chunk, tokens=idx)
        for k, r in (("logp", lp), ("entropy", en), ("lse", ls)):
            v = valid[idx]
            assert_stats_close(got[k][idx][v], r[v], f"{what} {k}")
        dh_r, dW_r = O.backward(h, W, t, chunk, g_l, g_e, tokens=idx)
        assert_grad_close(got["dh"][idx], dh_r, f"{what} dh rows {a}..")
        ref_dW += dW_r
        log(f"[parity] {what}: oracle through token {idx[-1] + 1} of {N}")
    rw = assert_grad_close(got["dW"], ref_dW, f"{what} dW")
    log(f"[parity] {what}: dW frob {rw:.2e}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("workload_no,chunk", [(3, 512), (4, 1024), (4, 4096), (5, 4096)])
def test_parity_workload_sampled(workload_no, chunk):
    """Full-size workloads: all outputs computed on the GPU, the oracle
    evaluates 1,024 sampled tokens (plus masked samples) one by one; dW is
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
    idx = sample_tokens(t, 1024, seed=workload_no, include_masked=32)
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


def _peaked_case(seed, N, H, V, w_std, n_planted, n_high_row=1):
    """Logits of std about w_std * sqrt(H) (7 to 13 here); n_planted tokens
    whose hidden row points along their target's W row, half of them so that
    the target logit is about +30 above the rest and its probability rounds
    to 1 in float32, half at +8 (probabilities 0.01 to 0.5); n_high_row
    tokens whose every logit is shifted by about +80 (a common component of
    all W rows that only these tokens see). Masked tokens included."""
    rng = np.random.default_rng(seed)
    hf = rng.standard_normal((N, H)).astype(np.float32)
    Wf = (rng.standard_normal((V, H)) * w_std).astype(np.float32)
    Wf[:, 0] = 4.0 + rng.standard_normal(V).astype(np.float32) * np.float32(w_std)   # common component
    hf[:, 0] = 0.0
    t = rng.integers(0, V, size=N).astype(np.int32)
    planted = rng.choice(N, size=n_planted, replace=False)
    for k, i in enumerate(planted):
        w = Wf[t[i]].copy()
        w[0] = 0.0
        margin = 30.0 if k % 2 == 0 else 8.0
        hf[i] = (0.15 * hf[i] + margin * w / float(np.dot(w, w))).astype(np.float32)
        hf[i, 0] = 0.0
    rest = np.setdiff1d(np.arange(N), planted)
    high = rng.choice(rest, size=n_high_row, replace=False)
    hf[high, 0] = 20.0                     # + ~80 on every logit of these tokens
    masked = rng.choice(np.setdiff1d(rest, high), size=max(1, N // 64), replace=False)
    t[masked] = -1
    h = f32_to_bf16_bits(hf)
    W = f32_to_bf16_bits(Wf)
    g_l = rng.standard_normal(N).astype(np.float32)
    g_e = (rng.standard_normal(N) * 0.1).astype(np.float32)
    return h, W, t, g_l, g_e, planted, high


@pytest.mark.parametrize("w_std,T", [(0.5, 1.0), (1.0, 1.0), (0.5, 0.25)])
def test_parity_peaked_logits_full(w_std, T):
    """Peaked logits compared in full: target probabilities that round to 1
    (onehot - p cancels), logits of std 8 to 16 (64 at T = 0.25) feeding the
    running-max rescale, a row of logits near +80, near-zero entropies."""
    N, H, V, C = 640, 256, 4096, 128
    h, W, t, g_l, g_e, planted, high = _peaked_case(int(w_std * 100) + int(100 * T), N, H, V, w_std, 128)
    log(f"[parity] peaked logits w_std={w_std} T={T}")
    got = run_head(h, W, t, C, g_l, g_e, temperature=T)
    ref = O.forward_backward(h, W, t, C, g_l, g_e, temperature=T)
    valid = t >= 0
    for k in ("logp", "entropy", "lse"):
        assert_stats_close(got[k][valid], ref[k][valid], f"peaked {k}")
        assert np.all(got[k][~valid] == 0.0), f"peaked masked {k}"
    # the planted targets dominate: probability near 1, entropy near 0
    p_t = np.exp(ref["logp"][planted[::2]])
    assert np.all(p_t > 0.9999), "planted targets are saturated"
    assert np.all(ref["lse"][high] > 60.0), "the high row's lse"
    assert np.all(got["dh"][~valid] == 0.0)
    rh = assert_grad_close(got["dh"], ref["dh"], "peaked dh")
    rw = assert_grad_close(got["dW"], ref["dW"], "peaked dW")
    log(f"[parity] peaked w_std={w_std} T={T}: dh frob {rh:.2e}, dW frob {rw:.2e}")


@pytest.mark.timeout(600)
def test_parity_peaked_logits_workload2_shape():
    """Peaked logits at the one-sequence shape (N 4096, H 2560, V 151936,
    chunk 512): logit std about 10, a quarter of the tokens planted, the
    oracle on 512 sampled tokens (planted, high-row and masked ones among
    them) with dW from cotangents vanishing outside the sample."""
    cfg = WORKLOADS[2]
    N, H, V, C = cfg.N, cfg.H, cfg.V, cfg.chunk_size
    log("[parity] peaked logits at the one-sequence shape: generating")
    h, W, t, g_l, g_e, planted, high = _peaked_case(2002, N, H, V, 0.2, N // 4, n_high_row=4)
    got = run_head(h, W, t, C, g_l, g_e)
    valid = t >= 0
    for k in ("logp", "entropy", "lse"):
        assert np.all(got[k][~valid] == 0.0) and np.all(np.isfinite(got[k])), k
    rng = np.random.default_rng(9)
    idx = np.unique(np.concatenate([rng.choice(np.flatnonzero(valid), 448, replace=False), planted[:32], high,
                                    np.flatnonzero(~valid)[:28]]))
    log(f"[parity] peaked one-sequence shape: oracle on {idx.size} tokens")
    ref_lp, ref_en, ref_lse = O.forward(h, W, t, C, tokens=idx)
    for k, ref in (("logp", ref_lp), ("entropy", ref_en), ("lse", ref_lse)):
        assert_stats_close(got[k][idx], ref, f"peaked one-sequence {k}")
    sl = np.zeros_like(g_l)
    se = np.zeros_like(g_e)
    sl[idx], se[idx] = g_l[idx], g_e[idx]
    ref_dh, ref_dW = O.backward(h, W, t, C, sl, se, tokens=idx)
    assert_grad_close(got["dh"][idx], ref_dh, "peaked one-sequence dh (sampled rows)")
    sparse = run_head(h, W, t, C, sl, se)
    assert_grad_close(sparse["dW"], ref_dW, "peaked one-sequence dW (sparse cotangents)")
