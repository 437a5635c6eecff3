"""Properties of the HIP path that hold at any size, through the C ABI:
determinism, chunk-size (in)variance, masking with non-finite hidden rows,
the optional entropy, the log-prob-only backward, empty inputs, streams."""
import json
import os

import numpy as np
import pytest

import oracle.lmhead_oracle as O
from gpu_common import assert_grad_close, assert_stats_close, dev, dev_bits, log, run_head
from synthetic import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


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


def test_bitwise_deterministic():
    """Two runs give identical bits: fixed reduction orders (the only atomics
    pick which workgroup computes a cotangent tile, which does not change the
    tile's values)."""
    h, W, t, g_l, g_e = _case(1, 1100, 256, 5000, n_masked=30)
    log("[props] determinism")
    a = run_head(h, W, t, 64, g_l, g_e)
    b = run_head(h, W, t, 64, g_l, g_e)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_chunk_size_changes_only_gradient_summation_order():
    """Per-token forward values are bitwise independent of chunk_size (the
    forward has no chunk-shaped transient); gradients differ only by float32
    summation order (google/tunix #2876: chunk 4096 vs 1024 within f32
    summation order)."""
    f = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))["chunk_4096_vs_1024_numerics"]
    h, W, t, g_l, g_e = _case(2, 1500, 256, 6000, n_masked=20)
    log("[props] chunk sizes")
    runs = {C: run_head(h, W, t, C, g_l, g_e) for C in (1, 37, 256, 1024, 4096)}
    ref = runs[4096]
    for C, r in runs.items():
        for k in ("logp", "entropy", "lse"):
            assert np.array_equal(r[k], ref[k]), (C, k)
        for k in ("dh", "dW"):
            scale = np.abs(ref[k]).max()
            diff = np.abs(r[k] - ref[k]).max()
            # pages' figure: 6.5e-5 on a gradient of max 83 (7.8e-7 relative)
            assert diff <= max(50 * f["max_abs_diff_grad"] / f["grad_max_abs"], 1e-5) * scale, (C, k, diff / scale)


def test_nonfinite_hidden_at_masked_positions_changes_nothing():
    """NaN / +-inf hidden rows at masked positions leave every output bit
    unchanged (tunix #2913 tests non-finite hidden states at masked
    positions)."""
    h, W, t, g_l, g_e = _case(3, 600, 128, 2000)
    t[[5, 77, 300, 599]] = [-1, 2000, -9, -1]
    log("[props] non-finite masked hidden")
    a = run_head(h, W, t, 100, g_l, g_e)
    h2 = h.copy()
    h2[5] = 0x7FC0       # NaN
    h2[77] = 0x7F80      # +inf
    h2[300, ::2] = 0xFF80  # -inf
    h2[599] = 0x7FC1
    b = run_head(h2, W, t, 100, g_l, g_e)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    for k in ("logp", "entropy", "lse"):
        assert np.all(a[k][[5, 77, 300, 599]] == 0.0)
    assert np.all(a["dh"][[5, 77, 300, 599]] == 0.0)
    assert np.all(np.isfinite(a["dW"]))


def test_entropy_optional_and_logprob_only_backward():
    """Forward without entropy gives the same logp / lse; the backward with
    only a log-prob cotangent (GRPO case: no entropy, no g_ent) matches the
    oracle with g_ent = 0."""
    h, W, t, g_l, _ = _case(4, 700, 192, 3001, n_masked=11)
    log("[props] entropy optional / GRPO backward")
    full = run_head(h, W, t, 128, g_l, None, with_entropy=True, backward=False)
    part = run_head(h, W, t, 128, g_l, None, with_entropy=False, backward=True, entropy_grad=False)
    assert part["entropy"] is None
    assert np.array_equal(full["logp"], part["logp"]) and np.array_equal(full["lse"], part["lse"])
    ref = O.forward_backward(h, W, t, 128, g_l, None)
    valid = t >= 0
    assert_stats_close(part["logp"][valid], ref["logp"][valid], "logp")
    assert_grad_close(part["dh"], ref["dh"], "dh (logp cotangent only)")
    assert_grad_close(part["dW"], ref["dW"], "dW (logp cotangent only)")


def test_entropy_cotangent_only_backward():
    """g_logp absent (zeros) and only an entropy cotangent: the entropy term
    of dz alone."""
    h, W, t, _, g_e = _case(5, 400, 128, 1500, n_masked=4)
    g_e = g_e * 10
    log("[props] entropy-only backward")
    import cross_entropy_amd as lm
    hd, Wd, td = dev_bits(h), dev_bits(W), dev(t)
    logp, ent, lse = lm.forward(hd, Wd, td, 64)
    dh, dW = lm.backward(hd, Wd, td, 64, lse, ent, None, dev(g_e))
    ref = O.forward_backward(h, W, t, 64, None, g_e)
    assert_grad_close(dh.cpu().numpy(), ref["dh"], "dh (entropy cotangent only)")
    assert_grad_close(dW.cpu().numpy(), ref["dW"], "dW (entropy cotangent only)")


def test_empty_and_all_masked():
    import torch
    import cross_entropy_amd as lm
    log("[props] empty and all-masked")
    H, V = 128, 700
    W_bits = f32_to_bf16_bits(np.random.default_rng(6).standard_normal((V, H)).astype(np.float32))
    W = dev_bits(W_bits)
    h0 = torch.zeros((0, H), dtype=torch.int16, device="cuda")
    t0 = torch.zeros((0,), dtype=torch.int32, device="cuda")
    logp, ent, lse = lm.forward(h0, W, t0, 16)
    assert logp.numel() == 0
    dh, dW = lm.backward(h0, W, t0, 16, lse, ent, logp, ent)
    torch.cuda.synchronize()
    assert dW.shape == (V, H) and bool((dW == 0).all())
    # every token masked: all outputs zero, dW zero
    h, _, _, g_l, g_e = _case(7, 300, H, V)
    t = np.full(300, -1, dtype=np.int32)
    t[::2] = V + 5
    r = run_head(h, W_bits, t, 50, g_l, g_e)
    for k in r:
        assert np.all(r[k] == 0.0), k


def test_runs_on_a_non_default_stream_and_reuses_one_workspace():
    import torch
    import cross_entropy_amd as lm
    h, W, t, g_l, g_e = _case(8, 520, 256, 2100, n_masked=7)
    log("[props] side stream + shared workspace")
    ref = run_head(h, W, t, 64, g_l, g_e)
    hd, Wd, td, gl, ge = dev_bits(h), dev_bits(W), dev(t), dev(g_l), dev(g_e)
    ws = lm.workspace_for(hd, Wd, 64, with_backward=True)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        logp, ent, lse = lm.forward(hd, Wd, td, 64, workspace=ws, stream=side)
        dh, dW = lm.backward(hd, Wd, td, 64, lse, ent, gl, ge, workspace=ws, stream=side)
    side.synchronize()
    for k, v in (("logp", logp), ("entropy", ent), ("lse", lse), ("dh", dh), ("dW", dW)):
        assert np.array_equal(v.cpu().numpy(), ref[k]), k


def test_concurrent_calls_from_threads_on_their_own_streams():
    """The library keeps no state between calls: four host threads, each
    with its own stream and workspace, run forward + backward on different
    inputs at the same time (their kernels interleave on the GPU); every
    output equals the same call made alone, bit for bit."""
    import threading
    import torch
    import cross_entropy_amd as lm
    shapes = [(900, 256, 3001, 64), (1500, 128, 5000, 512), (333, 320, 777, 7), (2048, 192, 2500, 300)]
    cases = [_case(40 + k, N, H, V, n_masked=N // 20) for k, (N, H, V, C) in enumerate(shapes)]
    log("[props] four threads on four streams")
    refs = [run_head(h, W, t, C, g_l, g_e) for (h, W, t, g_l, g_e), (_, _, _, C) in zip(cases, shapes)]
    dev_in = [(dev_bits(h), dev_bits(W), dev(t), dev(g_l), dev(g_e)) for h, W, t, g_l, g_e in cases]
    torch.cuda.synchronize()
    outs = [None] * len(cases)
    errors = []
    start = threading.Barrier(len(cases))

    def worker(k):
        try:
            hd, Wd, td, gl, ge = dev_in[k]
            C = shapes[k][3]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                ws = lm.workspace_for(hd, Wd, C, with_backward=True)
                start.wait()
                for _ in range(3):
                    logp, ent, lse = lm.forward(hd, Wd, td, C, workspace=ws, stream=s)
                    dh, dW = lm.backward(hd, Wd, td, C, lse, ent, gl, ge, workspace=ws, stream=s)
                s.synchronize()
            outs[k] = {"logp": logp, "entropy": ent, "lse": lse, "dh": dh, "dW": dW}
        except Exception as e:   # reported from the main thread
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(len(cases))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for k, (ref, got) in enumerate(zip(refs, outs)):
        for name, v in got.items():
            assert np.array_equal(v.cpu().numpy(), ref[name]), (k, name)


def test_backward_twice_on_one_workspace():
    """The backward's per-launch tile counters live in the workspace and are
    reset by each call: a second backward on the same (now dirty) workspace
    gives the same bits, on a shape with many cotangent tiles per launch."""
    import torch
    import cross_entropy_amd as lm
    h, W, t, g_l, g_e = _case(11, 2304, 256, 9000, n_masked=25)
    log("[props] backward twice on one workspace")
    hd, Wd, td, gl, ge = dev_bits(h), dev_bits(W), dev(t), dev(g_l), dev(g_e)
    ws = lm.workspace_for(hd, Wd, 1024, with_backward=True)
    logp, ent, lse = lm.forward(hd, Wd, td, 1024, workspace=ws)
    dh1, dW1 = lm.backward(hd, Wd, td, 1024, lse, ent, gl, ge, workspace=ws)
    dh2, dW2 = lm.backward(hd, Wd, td, 1024, lse, ent, gl, ge, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(dh1, dh2) and torch.equal(dW1, dW2)
    ref = run_head(h, W, t, 1024, g_l, g_e)
    assert np.array_equal(dh1.cpu().numpy(), ref["dh"]) and np.array_equal(dW1.cpu().numpy(), ref["dW"])


def _rel_fro(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30)


def test_token_permutation_is_exact():
    """Each token's logits, statistics and dh row are computed in an order
    that does not depend on where the token sits: permuting the tokens
    permutes logp, entropy, lse and the rows of dh bit for bit. dW sums over
    tokens, so only its float32 summation order changes."""
    h, W, t, g_l, g_e = _case(12, 1100, 256, 3000, n_masked=15)
    perm = np.random.default_rng(12).permutation(h.shape[0])
    log("[props] token permutation")
    a = run_head(h, W, t, 128, g_l, g_e)
    b = run_head(h[perm], W, t[perm], 128, g_l[perm], g_e[perm])
    for k in ("logp", "entropy", "lse", "dh"):
        assert np.array_equal(b[k], a[k][perm]), k
    assert _rel_fro(b["dW"], a["dW"]) < 1e-5


def test_vocabulary_permutation_is_equivariant():
    """Permuting W's rows (targets remapped) gives the same statistics up to
    float32 summation order over the vocabulary and permutes dW's rows. The
    cotangent is rounded to bf16, so the last-bit differences of lse can flip
    a rare rounding: the gradients are compared at 2e-4 (relative Frobenius)."""
    h, W, t, g_l, g_e = _case(13, 700, 256, 2500, n_masked=11)
    V = W.shape[0]
    pv = np.random.default_rng(13).permutation(V)
    inv = np.empty(V, np.int64)
    inv[pv] = np.arange(V)
    t2 = np.where((t >= 0) & (t < V), inv[np.clip(t, 0, V - 1)], t).astype(np.int32)
    log("[props] vocabulary permutation")
    a = run_head(h, W, t, 256, g_l, g_e)
    b = run_head(h, W[pv], t2, 256, g_l, g_e)
    for k in ("logp", "entropy", "lse"):
        err = np.abs(b[k].astype(np.float64) - a[k])
        assert np.all(err <= 1e-5 + 1e-5 * np.abs(a[k])), (k, err.max())
    assert _rel_fro(b["dh"], a["dh"]) < 2e-4
    assert _rel_fro(b["dW"], a["dW"][pv]) < 2e-4
    masked = ~((t >= 0) & (t < V))
    for k in ("logp", "entropy", "lse", "dh"):
        assert not np.any(b[k][masked]), k


def test_hip_graph_capture_and_replay():
    """The forward and backward enqueue kernels only (no memset, no
    synchronisation, no allocation by the library), so both can be captured
    into one HIP graph. Each of several replays, with eager work and a
    synchronisation between them, gives the eager run's bits."""
    import torch
    import cross_entropy_amd as lm
    h, W, t, g_l, g_e = _case(14, 1300, 256, 4100, n_masked=9)
    log("[props] graph capture")
    hd, Wd, td, gl, ge = dev_bits(h), dev_bits(W), dev(t), dev(g_l), dev(g_e)
    ws = lm.workspace_for(hd, Wd, 512, with_backward=True)
    ref = run_head(h, W, t, 512, g_l, g_e)
    dh = torch.empty((h.shape[0], h.shape[1]), dtype=torch.float32, device="cuda")
    dW = torch.empty((W.shape[0], W.shape[1]), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):      # warm the binding up outside the capture
        lm.forward(hd, Wd, td, 512, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        logp, ent, lse = lm.forward(hd, Wd, td, 512, workspace=ws)
        lm.backward(hd, Wd, td, 512, lse, ent, gl, ge, workspace=ws, dh=dh, dW=dW)
    for rep in range(3):
        dh.fill_(float("nan"))
        dW.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in (("logp", logp), ("entropy", ent), ("lse", lse), ("dh", dh), ("dW", dW)):
            assert np.array_equal(v.cpu().numpy(), ref[k]), (rep, k)


def test_tracing_counts_launches():
    import cross_entropy_amd as lm
    from cross_entropy_amd import _native
    h, W, t, g_l, g_e = _case(9, 300, 128, 1000)
    _native.trace_enable(True)
    run_head(h, W, t, 32, g_l, g_e)
    tr = _native.trace_read()
    _native.trace_enable(False)
    assert tr["fwd_stats_kernel"]["launches"] == 1 and tr["fwd_merge_kernel"]["launches"] == 1
    assert tr["bwd_step_kernel"]["launches"] >= 2 and tr["transpose_kernel"]["launches"] == 1
    assert tr["pad_rows_kernel"]["launches"] == 1   # 1000 % 64 != 0: W's last rows are padded
    assert abs(tr["fwd_stats_kernel"]["flops"] - 2.0 * 300 * 128 * 1000) < 1.0
    # the backward's credited work: the dh and dW GEMMs, 4 N H V over its launches (the
    # logits recompute is executed, not counted); the bench's roofline.frac rests on it
    assert abs(tr["bwd_step_kernel"]["flops"] - 4.0 * 300 * 128 * 1000) < 1.0
    assert tr["fwd_stats_kernel"]["ms"] > 0.0
    _ = lm
