"""Framework integration on the GPU: the autograd front end and the backward
that adds into a trainer's gradient buffers, through the C ABI, against the
fp64 oracle and against the overwriting backward."""
import numpy as np
import pytest

import oracle.lmhead_oracle as O
from gpu_common import assert_grad_close, assert_stats_close, dev, dev_bits, log, run_head
from synthetic import f32_to_bf16_bits

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


@pytest.mark.parametrize("T,with_entropy", [(None, True), (0.7, True), (None, False)])
def test_autograd_front_end(T, with_entropy):
    """loss = sum g_l logp (+ sum g_e entropy); loss.backward() through
    lmhead_logps gives the oracle's dh and dW (in bf16, the inputs' dtype)."""
    import torch
    import cross_entropy_amd as lm
    h, W, t, g_l, g_e = _case(41, 300, 128, 1000, n_masked=11)
    log(f"[integration] autograd T={T} entropy={with_entropy}")
    hd = dev_bits(h).view(torch.bfloat16).clone().requires_grad_(True)
    Wd = dev_bits(W).view(torch.bfloat16).clone().requires_grad_(True)
    td = dev(t)
    out = lm.lmhead_logps(hd, Wd, td, 64, temperature=T, with_entropy=with_entropy)
    logp, ent = out if with_entropy else (out, None)
    loss = (logp * dev(g_l)).sum()
    if with_entropy:
        loss = loss + (ent * dev(g_e)).sum()
    loss.backward()
    torch.cuda.synchronize()
    Tv = 1.0 if T is None else T
    ref = O.forward_backward(h, W, t, 64, g_l, g_e if with_entropy else None, temperature=Tv)
    valid = t >= 0
    assert_stats_close(logp.detach().cpu().numpy()[valid], ref["logp"][valid], "autograd logp")
    if with_entropy:
        assert_stats_close(ent.detach().cpu().numpy()[valid], ref["entropy"][valid], "autograd entropy")
    assert hd.grad.dtype == torch.bfloat16 and Wd.grad.dtype == torch.bfloat16
    assert_grad_close(hd.grad.float().cpu().numpy(), ref["dh"], "autograd dh")
    assert_grad_close(Wd.grad.float().cpu().numpy(), ref["dW"], "autograd dW")


def test_backward_accumulates_into_buffers():
    """accumulate=True adds the gradient into dh / dW: previous + gradient up
    to float32 summation order; masked dh rows keep their previous values."""
    import torch
    import cross_entropy_amd as lm
    h, W, t, g_l, g_e = _case(42, 700, 256, 3001, n_masked=25)
    N, H = h.shape
    V = W.shape[0]
    log("[integration] accumulate into dh / dW")
    hd, Wd, td = dev_bits(h), dev_bits(W), dev(t)
    ws = lm.workspace_for(hd, Wd, 96, with_backward=True)
    logp, ent, lse = lm.forward(hd, Wd, td, 96, workspace=ws)
    gl, ge = dev(g_l), dev(g_e)
    dh0, dW0 = lm.backward(hd, Wd, td, 96, lse, ent, gl, ge, workspace=ws)
    rng = np.random.default_rng(5)
    prev_h = rng.standard_normal((N, H)).astype(np.float32)
    prev_W = rng.standard_normal((V, H)).astype(np.float32)
    dh, dW = dev(prev_h), dev(prev_W)
    lm.backward(hd, Wd, td, 96, lse, ent, gl, ge, workspace=ws, dh=dh, dW=dW, accumulate=True)
    torch.cuda.synchronize()
    g_h, g_W = dh0.cpu().numpy(), dW0.cpu().numpy()
    got_h, got_W = dh.cpu().numpy(), dW.cpu().numpy()
    valid = t >= 0
    assert np.array_equal(got_h[~valid], prev_h[~valid]), "masked dh rows must be left unchanged"
    for got, prev, g, name in ((got_h[valid], prev_h[valid], g_h[valid], "dh"), (got_W, prev_W, g_W, "dW")):
        err = np.abs(got.astype(np.float64) - (prev.astype(np.float64) + g))
        lim = 1e-5 * (np.abs(prev) + np.abs(g)) + 1e-6
        assert np.all(err <= lim), f"{name}: accumulate differs from previous + gradient by {err.max():.3e}"
    # a second accumulation adds the same gradient again
    lm.backward(hd, Wd, td, 96, lse, ent, gl, ge, workspace=ws, dh=dh, dW=dW, accumulate=True)
    torch.cuda.synchronize()
    err = np.abs(dW.cpu().numpy().astype(np.float64) - (prev_W + 2.0 * g_W))
    assert np.all(err <= 2e-5 * (np.abs(prev_W) + 2 * np.abs(g_W)) + 1e-6)


def test_accumulate_with_no_tokens_leaves_dW():
    import torch
    import cross_entropy_amd as lm
    H, V = 128, 500
    rng = np.random.default_rng(6)
    Wd = dev_bits(f32_to_bf16_bits((rng.standard_normal((V, H)) * 0.05).astype(np.float32)))
    hd = torch.empty((0, H), dtype=torch.int16, device="cuda")
    td = torch.empty((0,), dtype=torch.int32, device="cuda")
    prev = rng.standard_normal((V, H)).astype(np.float32)
    dW = dev(prev)
    dh = torch.empty((0, H), dtype=torch.float32, device="cuda")
    z = torch.empty((0,), dtype=torch.float32, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    lm.backward(hd, Wd, td, 8, z, None, z, None, workspace=ws, dh=dh, dW=dW, accumulate=True)
    torch.cuda.synchronize()
    assert np.array_equal(dW.cpu().numpy(), prev)
