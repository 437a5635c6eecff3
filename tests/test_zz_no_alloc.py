"""The allocation-free forward (lmhead_logps_fwd_noalloc) through the C ABI
against the workspace forward (lmhead_logps_fwd_temp) it shares its kernels
with: bit for bit, and both within the oracle's bar; two calls in a row on
the library's fixed scratch array, the second one smaller, so a smaller call
must not see what the larger one left there."""
import numpy as np
import pytest

import oracle.lmhead_oracle as O
from gpu_common import assert_stats_close, dev, dev_bits, log
from synthetic import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _inputs(seed, N, H, V, n_masked):
    rng = np.random.default_rng(seed)
    h = f32_to_bf16_bits(rng.standard_normal((N, H)).astype(np.float32))
    W = f32_to_bf16_bits((rng.standard_normal((V, H)) * 0.05).astype(np.float32))
    t = rng.integers(0, V, size=N).astype(np.int32)
    t[rng.choice(N, size=n_masked, replace=False)] = -1
    return h, W, t


def _both(h_bits, W_bits, t, C, T):
    import torch
    import cross_entropy_amd as lm
    h, W, tt = dev_bits(h_bits), dev_bits(W_bits), dev(t)
    N = t.size
    out = {}
    for kind in ("noalloc", "workspace"):
        logp = torch.full((N,), 7.0, device="cuda")
        ent = torch.full((N,), 7.0, device="cuda")
        lse = torch.full((N,), 7.0, device="cuda")
        if kind == "noalloc":
            lm.lmhead_logps_fwd_noalloc(h, W, tt, C, T, logp, ent, lse)
        else:
            ws = lm.workspace_for(h, W, C, with_backward=False)
            lm.lmhead_logps_fwd_temp(h, W, tt, C, T, logp, ent, lse, ws)
        torch.cuda.synchronize()
        out[kind] = {"logp": logp.cpu().numpy(), "entropy": ent.cpu().numpy(), "lse": lse.cpu().numpy()}
    return out


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_noalloc_forward_two_calls(T):
    import cross_entropy_amd as lm
    calls = [(71, 9000, 256, 5003, 64, 40), (72, 700, 128, 777, 16, 9)]
    for seed, N, H, V, C, n_masked in calls:
        need = lm.lmhead_logps_workspace_bytes(N, H, V, C, with_backward=False)
        log(f"[noalloc] T={T} N={N} H={H} V={V} C={C}: scratch {need} bytes")
        h, W, t = _inputs(seed, N, H, V, n_masked)
        got = _both(h, W, t, C, T)
        ref = O.forward(h, W, t, C, temperature=T)
        valid = t >= 0
        for k, r in zip(("logp", "entropy", "lse"), ref):
            a, b = got["noalloc"][k], got["workspace"][k]
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{k}: noalloc differs from fwd_temp"
            assert_stats_close(a[valid], r[valid], f"noalloc {k}")
            assert np.all(a[~valid] == 0.0), f"noalloc masked {k}"


def test_noalloc_forward_random_sequence():
    """A seeded sequence of calls of random sizes (larger and smaller in
    turn, with and without the entropy output, temperatures 0.7 to 1.3) on the
    one scratch array: each gives the workspace forward's bits."""
    import torch
    import cross_entropy_amd as lm
    rng = np.random.default_rng(2718)
    for call in range(10):
        N = int(rng.integers(1, 12000))
        H = 64 * int(rng.integers(1, 6))
        V = int(rng.integers(2, 9000))
        C = int(rng.integers(1, N + 100))
        T = (1.0, 0.7, 1.3)[call % 3]
        with_ent = call % 3 != 2
        log(f"[noalloc] call {call}: N={N} H={H} V={V} C={C} T={T} entropy={with_ent}")
        h_bits, W_bits, t = _inputs(800 + call, N, H, V, int(rng.integers(0, N // 4 + 1)))
        h, W, tt = dev_bits(h_bits), dev_bits(W_bits), dev(t)
        outs = []
        for kind in ("noalloc", "workspace"):
            logp = torch.full((N,), 7.0, device="cuda")
            ent = torch.full((N,), 7.0, device="cuda") if with_ent else None
            lse = torch.full((N,), 7.0, device="cuda")
            if kind == "noalloc":
                lm.lmhead_logps_fwd_noalloc(h, W, tt, C, T, logp, ent, lse)
            else:
                ws = lm.workspace_for(h, W, C, with_backward=False)
                lm.lmhead_logps_fwd_temp(h, W, tt, C, T, logp, ent, lse, ws)
            torch.cuda.synchronize()
            outs.append([x.cpu().numpy().view(np.uint32) for x in (logp, ent, lse) if x is not None])
        for a, b in zip(*outs):
            assert np.array_equal(a, b), f"call {call}: noalloc differs from fwd_temp"


def test_noalloc_forward_on_a_side_stream():
    """On a stream of its own (the library takes the scratch of the stream's
    device) the allocation-free forward gives the workspace forward's bits."""
    import torch
    import cross_entropy_amd as lm
    h_bits, W_bits, t = _inputs(75, 2000, 256, 3001, 13)
    h, W, tt = dev_bits(h_bits), dev_bits(W_bits), dev(t)
    N = t.size
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    a = [torch.empty(N, device="cuda") for _ in range(3)]
    b = [torch.empty(N, device="cuda") for _ in range(3)]
    ws = lm.workspace_for(h, W, 256, with_backward=False)
    with torch.cuda.stream(side):
        lm.lmhead_logps_fwd_noalloc(h, W, tt, 256, 1.0, *a, stream=side)
        lm.lmhead_logps_fwd_temp(h, W, tt, 256, 1.0, *b, ws, stream=side)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert np.array_equal(x.cpu().numpy().view(np.uint32), y.cpu().numpy().view(np.uint32))


def test_noalloc_rejects_beyond_its_scratch():
    """A call whose partial records exceed the fixed array fails on the host
    with LMH_ERR_WORKSPACE and writes nothing."""
    import torch
    import cross_entropy_amd as lm
    from cross_entropy_amd import _native as nat
    N, H, V, C = 600_000, 64, 151936, 512
    assert lm.lmhead_logps_workspace_bytes(N, H, V, C, with_backward=False) > nat.NOALLOC_SCRATCH_BYTES
    h = torch.zeros((N, H), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((V, H), dtype=torch.bfloat16, device="cuda")
    t = torch.zeros(N, dtype=torch.int32, device="cuda")
    logp = torch.full((N,), 3.0, device="cuda")
    lse = torch.full((N,), 3.0, device="cuda")
    with pytest.raises(lm.LmheadError) as e:
        lm.lmhead_logps_fwd_noalloc(h, W, t, C, 1.0, logp, None, lse)
    assert e.value.code == -4
    torch.cuda.synchronize()
    assert bool((logp == 3.0).all()) and bool((lse == 3.0).all())


def test_noalloc_forward_in_a_hip_graph():
    """The use it exists for: captured into a HIP graph (after one eager call,
    which looks its scratch address up), replayed several times with eager
    work and synchronisations between the replays; every replay gives the
    eager call's bits, also after a larger call has used the scratch."""
    import torch
    import cross_entropy_amd as lm
    h_bits, W_bits, t = _inputs(73, 1500, 256, 4100, 11)
    h, W, tt = dev_bits(h_bits), dev_bits(W_bits), dev(t)
    N = t.size
    logp = torch.empty(N, device="cuda")
    ent = torch.empty(N, device="cuda")
    lse = torch.empty(N, device="cuda")
    lm.lmhead_logps_fwd_noalloc(h, W, tt, 512, 0.7, logp, ent, lse)
    torch.cuda.synchronize()
    ref = [x.cpu().numpy().copy() for x in (logp, ent, lse)]
    big = _inputs(74, 9000, 256, 5003, 40)
    bh, bW, bt = dev_bits(big[0]), dev_bits(big[1]), dev(big[2])
    bl, be, bs = (torch.empty(9000, device="cuda") for _ in range(3))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    log("[noalloc] graph capture")
    with torch.cuda.graph(g, stream=side):
        lm.lmhead_logps_fwd_noalloc(h, W, tt, 512, 0.7, logp, ent, lse)
    for rep in range(3):
        for x in (logp, ent, lse):
            x.fill_(float("nan"))
        lm.lmhead_logps_fwd_noalloc(bh, bW, bt, 64, 1.0, bl, be, bs)   # other contents in the scratch
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, x, r in zip(("logp", "entropy", "lse"), (logp, ent, lse), ref):
            assert np.array_equal(x.cpu().numpy(), r), (rep, name)
