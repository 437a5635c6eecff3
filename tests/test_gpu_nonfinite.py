"""Non-finite logits in unmasked rows on the GPU against the fp64 oracle
(google/tunix pull request #2913 checks its fused scoring, and the cotangent
of its one-pass backward, on logits with inf, -inf and NaN entries and a row
of no finite logit). Reading: IEEE evaluation of the definitions with the
log-sum-exp shifted by the row max when finite and by 0 otherwise; in the
cotangent, the entropy term is formed only for a nonzero entropy cotangent
and an entry of probability 0 gets no probability term. NaN, +inf and -inf
must land exactly where the oracle puts them, in logp / entropy / lse and in
dh / dW, and the finite values must meet the usual bar."""
import numpy as np
import pytest

import oracle.lmhead_oracle as O
from gpu_common import ATOL, FROB, RTOL, frob_rel, log, run_head
from synthetic import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

POS_INF, NEG_INF, NAN = 0x7F80, 0xFF80, 0x7FC0


def _case(seed=31, N=300, H=128, V=1000):
    rng = np.random.default_rng(seed)
    hf = rng.standard_normal((N, H)).astype(np.float32)
    hf[:, 0] = np.abs(hf[:, 0]) + 0.25            # inf * h[:, 0] keeps the sign of inf
    h = f32_to_bf16_bits(hf)
    W = f32_to_bf16_bits((rng.standard_normal((V, H)) * 0.05).astype(np.float32))
    t = rng.integers(0, V, size=N).astype(np.int32)
    t[rng.choice(N, size=12, replace=False)] = -1
    return h, W, t


def _same(gpu, ref, what):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.array_equal(np.isnan(gpu), np.isnan(ref)), f"{what}: NaN positions differ"
    assert np.array_equal(np.isposinf(gpu), np.isposinf(ref)), f"{what}: +inf positions differ"
    assert np.array_equal(np.isneginf(gpu), np.isneginf(ref)), f"{what}: -inf positions differ"
    fin = np.isfinite(ref)
    err = np.abs(gpu[fin] - ref[fin])
    assert np.all(err <= ATOL + RTOL * np.abs(ref[fin])), f"{what}: finite values out of tolerance"


def _same_grad(gpu, ref, what):
    """Non-finite positions identical; the finite entries within the
    relative Frobenius bar (exactly 0 when the oracle's are all 0)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    for name, f in (("NaN", np.isnan), ("+inf", np.isposinf), ("-inf", np.isneginf)):
        bad = np.argwhere(f(gpu) != f(ref))
        assert bad.size == 0, f"{what}: {name} positions differ at {len(bad)} entries, first {bad[0].tolist()}"
    fin = np.isfinite(ref)
    r = frob_rel(gpu[fin], ref[fin])
    assert r <= FROB, f"{what}: finite entries' relative Frobenius error {r:.3e}"
    return r


def _special_row(W, v, bits):
    W = W.copy()
    W[v] = 0
    W[v, 0] = bits
    return W


@pytest.mark.parametrize("kind,bits", [("-inf entry", NEG_INF), ("+inf entry", POS_INF), ("NaN entry", NAN)])
def test_nonfinite_vocabulary_entry(kind, bits):
    h, W, t = _case()
    v = 777                        # in the ragged last vocabulary tile's live rows
    valid = t >= 0
    t[np.flatnonzero(valid)[:5]] = v   # a few tokens target the special entry
    Ws = _special_row(W, v, bits)
    log(f"[nonfinite] {kind}")
    got = run_head(h, Ws, t, 64, backward=True, g_l=np.ones(t.size, np.float32))
    ref = O.forward(h, Ws, t, 64)
    for k, r in zip(("logp", "entropy", "lse"), ref):
        _same(got[k], r, f"{kind} {k}")
        assert np.all(got[k][~valid] == 0.0), f"{kind}: masked {k}"
    assert np.all(got["dh"][~valid] == 0.0), f"{kind}: masked dh rows"


def test_row_of_no_finite_logit():
    h, W, t = _case(32)
    Wn = W.copy()
    Wn[:, 0] = f32_to_bf16_bits(-(np.abs(O.widen_bf16(W[:, 0])) + 0.125).astype(np.float32))
    hn = h.copy()
    rows = [3, 150, 299]
    t[rows] = [5, 0, 999]
    hn[rows] = 0
    hn[rows, 0] = POS_INF           # logits of these tokens: +inf * (negative) = -inf everywhere
    log("[nonfinite] rows of no finite logit")
    got = run_head(hn, Wn, t, 64, backward=False)
    ref = O.forward(hn, Wn, t, 64)
    for k, r in zip(("logp", "entropy", "lse"), ref):
        _same(got[k], r, f"no finite logit {k}")
    assert np.all(got["lse"][rows] == -np.inf) and np.all(np.isnan(got["logp"][rows]))
    # the other tokens are those of the finite head
    fine = np.setdiff1d(np.arange(t.size), rows)
    plain = run_head(h, Wn, t, 64, backward=False)
    for k in ("logp", "entropy", "lse"):
        assert np.array_equal(got[k][fine], plain[k][fine]), k


@pytest.mark.parametrize("v", [777, 100], ids=["ragged-tile", "full-tile"])
@pytest.mark.parametrize("g_ent_mode", ["none", "dense", "half-zero"])
@pytest.mark.parametrize("kind,bits", [("-inf", NEG_INF), ("+inf", POS_INF), ("NaN", NAN)])
def test_nonfinite_gradients(kind, bits, g_ent_mode, v):
    """dh and dW at a non-finite vocabulary entry against the oracle: with
    log-prob cotangents only, a -inf entry's column carries g_l at its
    targets and 0 elsewhere and the other gradients are those of the finite
    head (only dh's column through the -inf table entry is 0 * -inf = NaN);
    with entropy cotangents the NaN entropy reaches the entries of positive
    probability; half-zero entropy cotangents mix both in one wave."""
    h, W, t = _case(seed=41 + v)
    rng = np.random.default_rng(v)
    N = t.size
    valid = t >= 0
    t[np.flatnonzero(valid)[:4]] = v          # a few tokens target the special entry
    g_l = rng.standard_normal(N).astype(np.float32)
    if g_ent_mode == "none":
        g_e = None
    else:
        g_e = (rng.standard_normal(N) * 0.1).astype(np.float32)
        if g_ent_mode == "half-zero":
            g_e[::2] = 0.0
    Ws = _special_row(W, v, bits)
    log(f"[nonfinite] gradients: {kind} entry at {v}, g_ent {g_ent_mode}")
    got = run_head(h, Ws, t, 64, g_l, g_e, backward=True)
    ref_dh, ref_dW = O.backward(h, Ws, t, 64, g_l, g_e)
    assert np.all(got["dh"][~valid] == 0.0), "masked dh rows"
    rh = _same_grad(got["dh"], ref_dh, f"{kind} {g_ent_mode} dh")
    rw = _same_grad(got["dW"], ref_dW, f"{kind} {g_ent_mode} dW")
    if kind == "-inf" and g_ent_mode == "none":
        # the closed form: finite everywhere but dh's column through W[v] = -inf
        assert np.all(np.isfinite(got["dW"])) and np.all(np.isfinite(got["dh"][:, 1:]))
    log(f"[nonfinite] {kind} {g_ent_mode}: finite dh frob {rh:.2e}, dW frob {rw:.2e}")


def test_row_of_no_finite_logit_gradients():
    """A token whose logits are all -inf: lse = -inf, its cotangent NaN, so
    its dh row and every dW row (its hidden row holds +inf) are NaN; the
    masked rows stay 0."""
    h, W, t = _case(33)
    Wn = W.copy()
    Wn[:, 0] = f32_to_bf16_bits(-(np.abs(O.widen_bf16(W[:, 0])) + 0.125).astype(np.float32))
    hn = h.copy()
    rows = [7, 200]
    t[rows] = [5, 999]
    hn[rows] = 0
    hn[rows, 0] = POS_INF
    rng = np.random.default_rng(3)
    g_l = rng.standard_normal(t.size).astype(np.float32)
    log("[nonfinite] gradients: rows of no finite logit")
    got = run_head(hn, Wn, t, 64, g_l, None)
    ref_dh, ref_dW = O.backward(hn, Wn, t, 64, g_l, None)
    _same_grad(got["dh"], ref_dh, "no finite logit dh")
    _same_grad(got["dW"], ref_dW, "no finite logit dW")


@pytest.mark.parametrize("kind,bits", [("-inf", NEG_INF), ("+inf", POS_INF)])
def test_nonfinite_gradients_tempered(kind, bits):
    """The same readings at T = 0.7: the tempered cotangent divides by T,
    which moves no NaN or inf and scales the finite values."""
    h, W, t = _case(seed=45)
    rng = np.random.default_rng(7)
    valid = t >= 0
    t[np.flatnonzero(valid)[:4]] = 100
    g_l = rng.standard_normal(t.size).astype(np.float32)
    g_e = (rng.standard_normal(t.size) * 0.1).astype(np.float32)
    g_e[::3] = 0.0
    Ws = _special_row(W, 100, bits)
    log(f"[nonfinite] tempered gradients: {kind}")
    got = run_head(h, Ws, t, 64, g_l, g_e, backward=True, temperature=0.7)
    ref_dh, ref_dW = O.backward(h, Ws, t, 64, g_l, g_e, temperature=0.7)
    assert np.all(got["dh"][~valid] == 0.0)
    _same_grad(got["dh"], ref_dh, f"tempered {kind} dh")
    _same_grad(got["dW"], ref_dW, f"tempered {kind} dW")


@pytest.mark.parametrize("kind,bits", [("-inf", NEG_INF), ("NaN", NAN)])
def test_nonfinite_bf16_gradients(kind, bits):
    """The bf16-gradient backward at a non-finite entry: the same NaN and inf
    positions as the float32 backward, and its finite values rounded to bf16."""
    import torch
    import cross_entropy_amd as lm
    from gpu_common import dev, dev_bits
    h, W, t = _case(seed=46)
    rng = np.random.default_rng(8)
    valid = t >= 0
    t[np.flatnonzero(valid)[:4]] = 777
    g_l = rng.standard_normal(t.size).astype(np.float32)
    Ws = _special_row(W, 777, bits)
    hd, Wd, td = dev_bits(h), dev_bits(Ws), dev(t)
    logp, ent, lse = lm.forward(hd, Wd, td, 64)
    log(f"[nonfinite] bf16 gradients: {kind}")
    dh32, dW32 = lm.backward(hd, Wd, td, 64, lse, None, dev(g_l), None)
    dh16, dW16 = lm.backward(hd, Wd, td, 64, lse, None, dev(g_l), None, grad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for name, a32, a16 in (("dh", dh32, dh16), ("dW", dW32, dW16)):
        f = a32.cpu().numpy()
        b = a16.float().cpu().numpy()
        assert np.array_equal(np.isnan(f), np.isnan(b)), f"{name}: NaN positions"
        assert np.array_equal(np.isposinf(f), np.isposinf(b)) and np.array_equal(np.isneginf(f), np.isneginf(b))
        fin = np.isfinite(f)
        want = a32.to(torch.bfloat16).float().cpu().numpy()
        assert np.array_equal(want[fin], b[fin]), f"{name}: finite values are not the float32 ones rounded"
