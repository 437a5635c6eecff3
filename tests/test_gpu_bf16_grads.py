"""The backward writing bf16 gradients (lmhead_logps_bwd_bf16) through the C
ABI. Its float32 sums run in the same block order as the float32 backward's
and each element is rounded once, so its output must be the float32
backward's rounded to bf16 (nearest even), bit for bit, in both block orders
(vocabulary blocks outer when N <= V, token blocks outer otherwise), with
and without adding into the caller's bf16 gradients; and it must meet the
oracle's bar after the rounding."""
import numpy as np
import pytest

import oracle.lmhead_oracle as O
from gpu_common import assert_grad_close, dev, dev_bits, log
from synthetic import WORKLOADS, f32_to_bf16_bits, make_cotangents, make_inputs

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


def _both(h, W, t, C, g_l, g_e, T=1.0, prev=None):
    """The float32 and the bf16 backward on the same forward; with `prev`
    (bf16 dh, dW bit patterns) both add into it (the float32 one into its
    widened values). Returns numpy (f32 dh, f32 dW, bf16 dh bits, bf16 dW bits)."""
    import torch
    import cross_entropy_amd as lm
    from cross_entropy_amd import _native as nat
    hd, Wd, td = dev_bits(h), dev_bits(W), dev(t)
    N, H = h.shape
    V = W.shape[0]
    logp, ent, lse = lm.forward(hd, Wd, td, C, temperature=T)
    gl = dev(g_l)
    ge = None if g_e is None else dev(g_e)
    entp = ent if ge is not None else None
    flags = 0
    if prev is None:
        dh32 = torch.empty((N, H), dtype=torch.float32, device="cuda")
        dW32 = torch.empty((V, H), dtype=torch.float32, device="cuda")
        dh16 = torch.empty((N, H), dtype=torch.bfloat16, device="cuda")
        dW16 = torch.empty((V, H), dtype=torch.bfloat16, device="cuda")
    else:
        flags = nat.BWD_ACCUMULATE_DH | nat.BWD_ACCUMULATE_DW
        dh16 = dev_bits(prev[0]).view(torch.bfloat16).clone()
        dW16 = dev_bits(prev[1]).view(torch.bfloat16).clone()
        dh32 = dh16.float()
        dW32 = dW16.float()
    ws32 = lm.workspace_for(hd, Wd, C, with_backward=True)
    lm.lmhead_logps_bwd_ex(hd, Wd, td, C, T, lse, entp, gl, ge, dh32, dW32, flags, ws32)
    ws16 = lm.workspace_for(hd, Wd, C, with_backward="bf16")
    lm.lmhead_logps_bwd_bf16(hd, Wd, td, C, T, lse, entp, gl, ge, dh16, dW16, flags, ws16)
    torch.cuda.synchronize()
    return (dh32, dW32, dh16, dW16)


def _assert_rounded(f32, b16, what):
    import torch
    want = f32.to(torch.bfloat16).view(torch.int16).cpu().numpy()
    got = b16.view(torch.int16).cpu().numpy()
    bad = np.argwhere(want != got)
    assert bad.size == 0, f"{what}: {len(bad)} elements differ from the rounded float32 gradient, first {bad[0]}"


@pytest.mark.parametrize("N,H,V,C,n_masked,T,ent", [
    (700, 320, 3001, 7, 40, 1.0, True),       # N <= V: vocabulary blocks outer, 3 x 12 blocks
    (2100, 128, 777, 64, 30, 0.7, True),      # N > V: token blocks outer, many token blocks
    (2100, 128, 777, 64, 30, 1.0, False),     # the log-prob-only backward
    (513, 256, 4097, 4096, 5, 1.0, True),     # one block
    (1, 128, 777, 1, 0, 1.0, True),           # one token
    (64, 64, 5, 1, 3, 1.0, True),             # fewer vocabulary rows than an MFMA block
])
def test_bf16_gradients_are_the_float32_ones_rounded(N, H, V, C, n_masked, T, ent):
    h, W, t, g_l, g_e = _case(N + V, N, H, V, n_masked=n_masked)
    log(f"[bf16] N={N} H={H} V={V} C={C} T={T} entropy={ent}")
    dh32, dW32, dh16, dW16 = _both(h, W, t, C, g_l, g_e if ent else None, T)
    _assert_rounded(dh32, dh16, "dh")
    _assert_rounded(dW32, dW16, "dW")
    valid = t >= 0
    assert np.all(dh16.float().cpu().numpy()[~valid] == 0.0), "masked dh rows"


def test_bf16_gradients_random_shapes():
    """A seeded sweep of shapes on both sides of N = V (so both block
    orders), chunk sizes 1 to past N, temperatures, with and without the
    entropy cotangent and the accumulate flags: the bf16 gradients are the
    float32 ones rounded, bit for bit."""
    rng = np.random.default_rng(8086)
    for case in range(10):
        N = int(rng.integers(1, 2500))
        H = 64 * int(rng.integers(1, 6))
        V = int(rng.integers(2, 3000))
        C = int(rng.integers(1, N + 50))
        T = (1.0, 0.7, 1.3)[case % 3]
        ent = case % 4 != 3
        h, W, t, g_l, g_e = _case(900 + case, N, H, V, n_masked=int(rng.integers(0, N // 4 + 1)))
        prev = None
        if case % 2:
            prev = (f32_to_bf16_bits(rng.standard_normal((N, H)).astype(np.float32) * 1e-2),
                    f32_to_bf16_bits(rng.standard_normal((V, H)).astype(np.float32) * 1e-2))
        what = f"random {case}: N={N} H={H} V={V} C={C} T={T} entropy={ent} accumulate={prev is not None}"
        log(f"[bf16] {what}")
        dh32, dW32, dh16, dW16 = _both(h, W, t, C, g_l, g_e if ent else None, T, prev=prev)
        _assert_rounded(dh32, dh16, f"{what} dh")
        _assert_rounded(dW32, dW16, f"{what} dW")


@pytest.mark.parametrize("N,H,V,C", [(700, 320, 3001, 7), (2100, 128, 777, 64), (300, 128, 1000, 4096)])
def test_bf16_gradients_add_into_previous(N, H, V, C):
    """With the accumulate flags: the previous bf16 values, widened, start
    the float32 sums; masked dh rows keep their previous bits."""
    h, W, t, g_l, g_e = _case(N + 2 * V, N, H, V, n_masked=17)
    rng = np.random.default_rng(N)
    prev = (f32_to_bf16_bits(rng.standard_normal((N, H)).astype(np.float32) * 1e-2),
            f32_to_bf16_bits(rng.standard_normal((V, H)).astype(np.float32) * 1e-2))
    log(f"[bf16] accumulate N={N} H={H} V={V} C={C}")
    dh32, dW32, dh16, dW16 = _both(h, W, t, C, g_l, g_e, 1.0, prev=prev)
    _assert_rounded(dh32, dh16, "dh (accumulate)")
    _assert_rounded(dW32, dW16, "dW (accumulate)")
    import torch
    valid = t >= 0
    got = dh16.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got[~valid], prev[0][~valid]), "masked dh rows keep their previous values"


def test_bf16_gradients_against_the_oracle():
    """After rounding to bf16 the gradients still meet the 5e-3 Frobenius bar."""
    h, W, t, g_l, g_e = _case(77, 700, 256, 5000, n_masked=20)
    log("[bf16] against the oracle")
    _, _, dh16, dW16 = _both(h, W, t, 96, g_l, g_e, 0.7)
    ref_dh, ref_dW = O.backward(h, W, t, 96, g_l, g_e, temperature=0.7)
    rh = assert_grad_close(dh16.float().cpu().numpy(), ref_dh, "bf16 dh")
    rw = assert_grad_close(dW16.float().cpu().numpy(), ref_dW, "bf16 dW")
    log(f"[bf16] oracle: dh frob {rh:.2e}, dW frob {rw:.2e}")


@pytest.mark.parametrize("workload_no,chunk", [(2, 512), (3, 512), (4, 1024), (5, 4096)])
def test_bf16_gradients_full_size_workloads(workload_no, chunk):
    """The workloads at full size, each in the launch configuration the
    benchmark times (the one-sequence head; the 16 x 4096-token batch; the
    context-rank share at H 4096; the packed row with its padding at chunk
    4096): the bf16 gradients are the float32 ones rounded, bit for bit. The
    float32 gradients themselves are compared with the oracle by the parity
    tests."""
    import torch
    cfg = WORKLOADS[workload_no]
    h, W, t = make_inputs(cfg)
    g_l, g_e = make_cotangents(cfg)
    log(f"[bf16] workload {workload_no} chunk {chunk}")
    dh32, dW32, dh16, dW16 = _both(h, W, t, chunk, g_l, g_e)
    _assert_rounded(dh32, dh16, f"workload {workload_no} dh")
    _assert_rounded(dW32, dW16, f"workload {workload_no} dW")
    valid = (t >= 0) & (t < W.shape[0])
    assert np.all(dh16.float().cpu().numpy()[~valid] == 0.0), "masked dh rows"
    del dh32, dW32, dh16, dW16
    torch.cuda.empty_cache()


def test_autograd_gradients_are_the_float32_ones_rounded():
    """The autograd front end hands bf16 inputs their gradients from the bf16
    backward: the float32 backward's, rounded, bit for bit."""
    import torch
    import cross_entropy_amd as lm
    h, W, t, g_l, g_e = _case(43, 500, 128, 3000, n_masked=9)
    hd = dev_bits(h).view(torch.bfloat16).clone().requires_grad_(True)
    Wd = dev_bits(W).view(torch.bfloat16).clone().requires_grad_(True)
    td = dev(t)
    logp, ent = lm.lmhead_logps(hd, Wd, td, 64)
    ((logp * dev(g_l)).sum() + (ent * dev(g_e)).sum()).backward()
    dh32, dW32, _, _ = _both(h, W, t, 64, g_l, g_e)
    _assert_rounded(dh32, hd.grad, "autograd dh")
    _assert_rounded(dW32, Wd.grad, "autograd dW")


def test_bf16_no_tokens():
    """N = 0 writes dW = 0 (bf16), or leaves it with the accumulate flag."""
    import torch
    import cross_entropy_amd as lm
    from cross_entropy_amd import _native as nat
    H, V = 128, 500
    rng = np.random.default_rng(8)
    Wd = dev_bits(f32_to_bf16_bits((rng.standard_normal((V, H)) * 0.05).astype(np.float32)))
    hd = torch.empty((0, H), dtype=torch.int16, device="cuda")
    td = torch.empty((0,), dtype=torch.int32, device="cuda")
    z = torch.empty((0,), dtype=torch.float32, device="cuda")
    dh = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    dW = torch.full((V, H), 3.0, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    flags = nat.BWD_ACCUMULATE_DH | nat.BWD_ACCUMULATE_DW
    lm.lmhead_logps_bwd_bf16(hd, Wd, td, 8, 1.0, z, None, z, None, dh, dW, flags, ws)
    torch.cuda.synchronize()
    assert bool((dW == 3.0).all())
    lm.lmhead_logps_bwd_bf16(hd, Wd, td, 8, 1.0, z, None, z, None, dh, dW, 0, ws)
    torch.cuda.synchronize()
    assert bool((dW == 0.0).all())


def test_bf16_backward_in_a_hip_graph():
    """The forward and the bf16 backward captured into one HIP graph and
    replayed three times: every replay gives the eager run's bits."""
    import torch
    import cross_entropy_amd as lm
    h, W, t, g_l, g_e = _case(15, 1300, 256, 4100, n_masked=9)
    hd, Wd, td, gl, ge = dev_bits(h), dev_bits(W), dev(t), dev(g_l), dev(g_e)
    N, H = h.shape
    V = W.shape[0]
    ws = lm.workspace_for(hd, Wd, 96, with_backward="bf16")
    logp, ent, lse = lm.forward(hd, Wd, td, 96, workspace=ws)
    dh, dW = lm.backward(hd, Wd, td, 96, lse, ent, gl, ge, workspace=ws, grad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = [x.view(torch.int16).cpu().numpy().copy() for x in (dh, dW)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    log("[bf16] graph capture")
    with torch.cuda.graph(g, stream=side):
        lm.lmhead_logps_fwd(hd, Wd, td, 96, logp, ent, lse, ws)
        lm.lmhead_logps_bwd_bf16(hd, Wd, td, 96, 1.0, lse, ent, gl, ge, dh, dW, 0, ws)
    for rep in range(3):
        dh.fill_(float("nan"))
        dW.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, x, r in (("dh", dh, ref[0]), ("dW", dW, ref[1])):
            assert np.array_equal(x.view(torch.int16).cpu().numpy(), r), (rep, name)


def test_autograd_memory_at_the_one_sequence_shape():
    """Between forward and backward the autograd front end holds the outputs,
    lse and nothing backward-sized (the forward's workspace is the split
    records only); the backward's peak allocation stays below what a float32
    dW [V, H] alone would take (1.56 GB here): the bf16 backward's float32
    accumulators cover min(N, V) x H plus one block's rows, and the gradients
    are bf16 from the start."""
    import torch
    import cross_entropy_amd as lm
    cfg = WORKLOADS[2]
    h, W, t = make_inputs(cfg)
    g_l, g_e = make_cotangents(cfg)
    N, H, V, C = cfg.N, cfg.H, cfg.V, cfg.chunk_size
    hd = dev_bits(h).view(torch.bfloat16).clone().requires_grad_(True)
    Wd = dev_bits(W).view(torch.bfloat16).clone().requires_grad_(True)
    td, gl, ge = dev(t), dev(g_l), dev(g_e)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    logp, ent = lm.lmhead_logps(hd, Wd, td, C)
    loss = (logp * gl).sum() + (ent * ge).sum()
    torch.cuda.synchronize()
    held = torch.cuda.memory_allocated() - base
    log(f"[bf16] autograd: held between forward and backward {held / 1e6:.1f} MB")
    assert held < 16 * N + (8 << 20), "only per-token outputs and lse are held"
    torch.cuda.reset_peak_memory_stats()
    before = torch.cuda.memory_allocated()
    loss.backward()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - before
    f32_dW = 4 * V * H
    ws = lm.lmhead_logps_workspace_bytes(N, H, V, C, with_backward="bf16")
    log(f"[bf16] autograd: backward peak {peak / 1e6:.1f} MB (workspace {ws / 1e6:.1f} MB, f32 dW {f32_dW / 1e6:.1f} MB)")
    assert peak < f32_dW, "no float32 [V, H] gradient"
    assert peak <= ws + 2 * (N + V) * H + (64 << 20)
    assert hd.grad.dtype == torch.bfloat16 and Wd.grad.dtype == torch.bfloat16
