"""Pins of the fp64 oracle: checks against what the mathematics fixes.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
a closed form, an invariant, the 50-digit brute force or a central finite
difference. ``tests/test_oracle.py`` runs them on the oracle as written, and
``tests/test_oracle_mutants.py`` shows that each plausible mistake planted in
the oracle (on the CPU) makes at least one of them fail.
"""
from __future__ import annotations

import math

import numpy as np

import oracle.lmhead_oracle as O
from oracle import bruteforce as B
from synthetic import f32_to_bf16_bits


def bf16(x) -> np.ndarray:
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def f64(bits) -> np.ndarray:
    return O.widen_bf16(bits)


def _rand_case(seed, N, H, V, h_std=1.0, w_std=0.5, n_masked=0):
    rng = np.random.default_rng(seed)
    h = bf16(rng.standard_normal((N, H)) * h_std)
    W = bf16(rng.standard_normal((V, H)) * w_std)
    t = rng.integers(0, V, size=N).astype(np.int32)
    if n_masked:
        t[rng.choice(N, size=n_masked, replace=False)] = -1
    g_l = rng.standard_normal(N)
    g_e = rng.standard_normal(N) * 0.3
    return h, W, t, g_l, g_e


def _close(a, b, rtol, atol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.abs(a - b)
    lim = atol + rtol * np.abs(b)
    assert np.all(err <= lim), f"{what}: max err {float(err.max()):.3e} (limit at worst {float(lim.flat[int(np.argmax(err - lim))]):.3e})"


# --- closed forms -----------------------------------------------------------------

def pin_W_zero():
    """W = 0: every logit is 0, so lse = ln V, logp = -ln V, entropy = ln V,
    dh = 0 and dW[v] = sum_i g_l,i (delta(v, t_i) - 1/V) h_i (the entropy
    term vanishes where p is uniform, since log p + entropy = 0)."""
    N, H, V = 6, 8, 11
    h, _, t, g_l, g_e = _rand_case(1, N, H, V)
    W = bf16(np.zeros((V, H)))
    logp, ent, lse = O.forward(h, W, t, chunk_size=4)
    _close(lse, np.full(N, math.log(V)), 1e-15, what="lse at W=0")
    _close(logp, np.full(N, -math.log(V)), 1e-15, what="logp at W=0")
    _close(ent, np.full(N, math.log(V)), 1e-14, what="entropy at W=0")
    dh, dW = O.backward(h, W, t, 4, g_l, g_e)
    assert np.all(np.abs(dh) <= 1e-15), "dh at W=0"
    hf = f64(h)
    want = np.zeros((V, H))
    for i in range(N):
        coef = -g_l[i] / V * np.ones(V)
        coef[t[i]] += g_l[i]
        want += np.outer(coef, hf[i])
    _close(dW, want, 1e-12, 1e-13, what="dW at W=0")


def pin_h_zero():
    """h = 0: same statistics as W = 0, dW = 0 and
    dh_i = g_l,i (W[t_i] - mean_v W[v])."""
    N, H, V = 5, 6, 9
    _, W, t, g_l, g_e = _rand_case(2, N, H, V)
    h = bf16(np.zeros((N, H)))
    logp, ent, lse = O.forward(h, W, t, chunk_size=2)
    _close(lse, np.full(N, math.log(V)), 1e-15, what="lse at h=0")
    _close(logp, np.full(N, -math.log(V)), 1e-15, what="logp at h=0")
    _close(ent, np.full(N, math.log(V)), 1e-14, what="entropy at h=0")
    dh, dW = O.backward(h, W, t, 2, g_l, g_e)
    assert np.all(dW == 0.0), "dW at h=0"
    Wf = f64(W)
    want = np.stack([g_l[i] * (Wf[t[i]] - Wf.mean(axis=0)) for i in range(N)])
    _close(dh, want, 1e-12, 1e-14, what="dh at h=0")


def pin_V1():
    """V = 1: logp = 0, entropy = 0, lse = z (the one logit), gradients 0."""
    N, H = 4, 5
    h, W, _, g_l, g_e = _rand_case(3, N, H, 1)
    t = np.zeros(N, dtype=np.int32)
    logp, ent, lse = O.forward(h, W, t, 3)
    z = f64(h) @ f64(W)[0]
    _close(lse, z, 1e-14, 1e-15, what="lse at V=1")
    assert np.all(np.abs(logp) <= 1e-15) and np.all(np.abs(ent) <= 1e-15), "V=1 logp/entropy"
    dh, dW = O.backward(h, W, t, 3, g_l, g_e)
    assert np.all(np.abs(dh) <= 1e-14) and np.all(np.abs(dW) <= 1e-14), "V=1 gradients"


def pin_V2():
    """V = 2: logp_t = -log(1 + exp(z_o - z_t)); entropy is the binary
    entropy of sigmoid(z_0 - z_1)."""
    N, H = 7, 4
    h, W, t, _, _ = _rand_case(4, N, H, 2, w_std=1.0)
    logp, ent, _ = O.forward(h, W, t, 7)
    z = f64(h) @ f64(W).T
    for i in range(N):
        zt, zo = z[i, t[i]], z[i, 1 - t[i]]
        want_lp = -math.log1p(math.exp(zo - zt))
        p0 = 1.0 / (1.0 + math.exp(z[i, 1] - z[i, 0]))
        want_h = -(p0 * math.log(p0) + (1 - p0) * math.log(1 - p0))
        _close(logp[i], want_lp, 1e-13, 1e-15, what="logp at V=2")
        _close(ent[i], want_h, 1e-13, 1e-15, what="entropy at V=2")


# --- brute force ------------------------------------------------------------------

def _bruteforce_case():
    N, H, V = 3, 4, 6
    h, W, t, g_l, g_e = _rand_case(5, N, H, V, h_std=1.0, w_std=0.7)
    t[1] = -1                      # one masked token
    return h, W, t, g_l, g_e


def pin_bruteforce_forward():
    """fp64 oracle vs 50-digit unshifted definitions on a tiny case."""
    h, W, t, _, _ = _bruteforce_case()
    logp, ent, lse = O.forward(h, W, t, 2)
    ref = B.forward(h.tolist(), W.tolist(), t.tolist())
    for i, (lp, en, ls) in enumerate(ref):
        _close(logp[i], float(lp), 1e-13, 1e-15, what=f"logp[{i}] vs brute force")
        _close(ent[i], float(en), 1e-13, 1e-15, what=f"entropy[{i}] vs brute force")
        _close(lse[i], float(ls), 1e-13, 1e-15, what=f"lse[{i}] vs brute force")


def pin_bruteforce_gradients():
    """fp64 oracle backward vs 50-digit central differences of L."""
    h, W, t, g_l, g_e = _bruteforce_case()
    dh, dW = O.backward(h, W, t, 2, g_l, g_e)
    rdh, rdW = B.gradients(h.tolist(), W.tolist(), t.tolist(), g_l, g_e)
    rdh = np.array([[float(x) for x in row] for row in rdh])
    rdW = np.array([[float(x) for x in row] for row in rdW])
    scale_h = max(1e-300, np.abs(rdh).max())
    scale_W = max(1e-300, np.abs(rdW).max())
    _close(dh, rdh, 1e-11, 1e-13 * scale_h, what="dh vs brute-force differences")
    _close(dW, rdW, 1e-11, 1e-13 * scale_W, what="dW vs brute-force differences")


def pin_fd_gradients():
    """fp64 central differences of L (on float64 inputs) vs the backward, on a
    case with a masked token and a partial last chunk."""
    N, H, V = 5, 6, 7
    h, W, t, g_l, g_e = _rand_case(6, N, H, V, w_std=0.6)
    t[3] = -1
    hf, Wf = f64(h), f64(W)
    dh, dW = O.backward(h, W, t, 2, g_l, g_e)
    eps = 1e-6
    for mat, grad, name in ((hf, dh, "dh"), (Wf, dW, "dW")):
        num = np.zeros_like(mat)
        for idx in np.ndindex(mat.shape):
            keep = mat[idx]
            mat[idx] = keep + eps
            up = O.loss(hf, Wf, t, g_l, g_e)
            mat[idx] = keep - eps
            dn = O.loss(hf, Wf, t, g_l, g_e)
            mat[idx] = keep
            num[idx] = (up - dn) / (2 * eps)
        _close(grad, num, 1e-7, 1e-8, what=f"{name} vs central differences")


# --- invariants -------------------------------------------------------------------

def pin_normalisation():
    """sum_v p = 1 shows as sum_v dz = 0, hence sum_v dW[v, :] = 0;
    0 <= entropy <= ln V; logp <= 0."""
    N, H, V = 9, 7, 13
    h, W, t, g_l, g_e = _rand_case(7, N, H, V, w_std=1.5)
    logp, ent, _ = O.forward(h, W, t, 4)
    assert np.all(logp <= 1e-15), "logp <= 0"
    assert np.all(ent >= -1e-15) and np.all(ent <= math.log(V) + 1e-12), "0 <= entropy <= ln V"
    _, dW = O.backward(h, W, t, 4, g_l, g_e)
    col = np.abs(dW.sum(axis=0))
    assert np.all(col <= 1e-12 * max(1.0, np.abs(dW).max())), f"sum_v dW = {col.max():.3e}"


def pin_shift_invariance():
    """Adding one row vector c to every row of W shifts every logit of token i
    by h_i . c: lse moves by h_i . c and nothing else changes. W and c are
    dyadic (k/64) so W + c is exact in bf16."""
    N, H, V = 6, 5, 8
    rng = np.random.default_rng(8)
    h = bf16(rng.integers(-64, 64, size=(N, H)) / 32.0)
    Wi = rng.integers(-40, 40, size=(V, H))
    ci = rng.integers(-20, 20, size=H)
    W = bf16(Wi / 64.0)
    W2 = bf16((Wi + ci[None, :]) / 64.0)
    t = rng.integers(0, V, size=N).astype(np.int32)
    g_l = rng.standard_normal(N)
    g_e = rng.standard_normal(N)
    a = O.forward_backward(h, W, t, 4, g_l, g_e)
    b = O.forward_backward(h, W2, t, 4, g_l, g_e)
    shift = f64(h) @ (ci / 64.0)
    _close(b["lse"], a["lse"] + shift, 1e-12, 1e-12, what="lse shift")
    _close(b["logp"], a["logp"], 1e-11, 1e-12, what="logp under shift")
    _close(b["entropy"], a["entropy"], 1e-11, 1e-12, what="entropy under shift")
    _close(b["dh"], a["dh"], 1e-9, 1e-11, what="dh under shift")
    _close(b["dW"], a["dW"], 1e-9, 1e-11, what="dW under shift")


def pin_masking():
    """Masked ids (-1, other negatives, >= V) give exactly 0 outputs and dh
    rows; NaN/inf hidden rows at masked positions change nothing; appending
    masked tokens leaves dW unchanged."""
    N, H, V = 8, 6, 10
    h, W, t, g_l, g_e = _rand_case(9, N, H, V)
    t[[1, 4, 6]] = [-1, V, -7]
    a = O.forward_backward(h, W, t, 3, g_l, g_e)
    for k in ("logp", "entropy", "lse"):
        assert np.all(a[k][[1, 4, 6]] == 0.0), f"masked {k}"
        assert np.all(a[k][[0, 2, 3, 5, 7]] != 0.0), f"unmasked {k} is zero"
    assert np.all(a["dh"][[1, 4, 6]] == 0.0), "masked dh rows"
    h2 = h.copy()
    h2[1] = 0x7FC0      # NaN
    h2[4] = 0x7F80      # +inf
    h2[6] = 0xFF80      # -inf
    b = O.forward_backward(h2, W, t, 3, g_l, g_e)
    for k in a:
        assert np.array_equal(a[k], b[k]), f"non-finite masked hidden changed {k}"
    h3 = np.concatenate([h, bf16(np.ones((3, H)))])
    t3 = np.concatenate([t, np.array([-1, -1, V + 3], dtype=np.int32)])
    c = O.backward(h3, W, t3, 3, np.concatenate([g_l, [1.0, 2.0, 3.0]]), np.concatenate([g_e, [1.0, 1.0, 1.0]]))
    _close(c[1], a["dW"], 1e-15, 1e-15, what="dW with appended masked tokens")
    # the unmasked tokens must match a run without any masked token
    keep = np.array([0, 2, 3, 5, 7])
    d = O.forward_backward(h[keep], W, t[keep], 3, g_l[keep], g_e[keep])
    for k in ("logp", "entropy", "lse"):
        _close(a[k][keep], d[k], 1e-13, 1e-15, what=f"unmasked {k} vs masked-free run")
    _close(a["dW"], d["dW"], 1e-12, 1e-14, what="dW vs masked-free run")


def pin_chunk_invariance():
    """Per-token values do not depend on chunk_size (1, a non-divisor, N, > N);
    dW agrees to float64 summation order."""
    N, H, V = 11, 5, 9
    h, W, t, g_l, g_e = _rand_case(10, N, H, V)
    t[2] = -1
    ref = O.forward_backward(h, W, t, N, g_l, g_e)
    for C in (1, 3, 4, 7, 64):
        got = O.forward_backward(h, W, t, C, g_l, g_e)
        for k in ("logp", "entropy", "lse", "dh"):
            _close(got[k], ref[k], 1e-14, 1e-15, what=f"{k} at chunk {C}")
        _close(got["dW"], ref["dW"], 1e-13, 1e-15, what=f"dW at chunk {C}")
    assert len(O.chunk_ranges(N, 4)) == 3 and O.chunk_ranges(N, 4)[-1] == (8, 11)


def pin_subset_evaluation():
    """The sampled evaluation used at full sizes: forward on a token subset
    equals the full forward on those tokens; the backward restricted to a
    subset equals the full backward when every other cotangent is zero."""
    N, H, V = 10, 4, 7
    h, W, t, g_l, g_e = _rand_case(11, N, H, V)
    t[5] = -1
    idx = np.array([1, 4, 5, 8])
    full = O.forward_backward(h, W, t, 3, g_l, g_e)
    sub = O.forward(h, W, t, 3, tokens=idx)
    for k, v in zip(("logp", "entropy", "lse"), sub):
        _close(v, full[k][idx], 1e-14, 1e-15, what=f"subset {k}")
    gl = np.zeros(N)
    ge = np.zeros(N)
    gl[idx], ge[idx] = g_l[idx], g_e[idx]
    sparse_full = O.backward(h, W, t, 3, gl, ge)
    dh_s, dW_s = O.backward(h, W, t, 3, gl, ge, tokens=idx)
    _close(dh_s, full["dh"][idx], 1e-14, 1e-15, what="subset dh")
    _close(dW_s, sparse_full[1], 1e-13, 1e-15, what="subset dW")


# --- temperature ------------------------------------------------------------------
# tunix #2913 tests its head at temperatures 1 and 0.7; the tempered head
# scores z / T and divides the backward's cotangent by T.

def _scaled_bits(bits, factor):
    return bf16(f64(bits) * factor)


def pin_temperature_power_of_two():
    """T = 2^k scores exactly what T = 1 scores with W scaled by 2^-k (exact in
    bf16 for normal values): same statistics and dh, and dW(T) = 2^-k dW(W 2^-k)
    by the chain rule through W / T."""
    h, W, t, g_l, g_e = _rand_case(11, 9, 8, 13, w_std=0.5, n_masked=2)
    for k in (1, -1, 3):
        T = 2.0 ** k
        Ws = _scaled_bits(W, 2.0 ** -k)
        assert np.array_equal(f64(Ws), f64(W) * 2.0 ** -k), "scaling by a power of two must be exact"
        a = O.forward_backward(h, W, t, 4, g_l, g_e, temperature=T)
        b = O.forward_backward(h, Ws, t, 4, g_l, g_e)
        for key in ("logp", "entropy", "lse", "dh"):
            _close(a[key], b[key], 1e-13, 1e-15, what=f"T={T} {key} vs scaled W")
        _close(a["dW"], b["dW"] * 2.0 ** -k, 1e-12, 1e-15, what=f"T={T} dW vs scaled W")


def pin_temperature_bruteforce():
    """T = 0.7: fp64 oracle vs the 50-digit unshifted definitions, forward and
    central-difference gradients."""
    h, W, t, g_l, g_e = _bruteforce_case()
    logp, ent, lse = O.forward(h, W, t, 2, temperature=0.7)
    ref = B.forward(h.tolist(), W.tolist(), t.tolist(), temperature="0.7")
    for i, (lp, en, ls) in enumerate(ref):
        _close(logp[i], float(lp), 1e-13, 1e-15, what=f"T=0.7 logp[{i}] vs brute force")
        _close(ent[i], float(en), 1e-13, 1e-15, what=f"T=0.7 entropy[{i}] vs brute force")
        _close(lse[i], float(ls), 1e-13, 1e-15, what=f"T=0.7 lse[{i}] vs brute force")
    dh, dW = O.backward(h, W, t, 2, g_l, g_e, temperature=0.7)
    rdh, rdW = B.gradients(h.tolist(), W.tolist(), t.tolist(), g_l, g_e, temperature="0.7")
    rdh = np.array([[float(x) for x in row] for row in rdh])
    rdW = np.array([[float(x) for x in row] for row in rdW])
    _close(dh, rdh, 1e-11, 1e-13 * np.abs(rdh).max(), what="T=0.7 dh vs brute-force differences")
    _close(dW, rdW, 1e-11, 1e-13 * np.abs(rdW).max(), what="T=0.7 dW vs brute-force differences")


def pin_temperature_fd():
    """T = 0.7: fp64 central differences of the tempered loss vs the backward."""
    N, H, V = 4, 5, 6
    h, W, t, g_l, g_e = _rand_case(12, N, H, V, w_std=0.6)
    t[2] = -1
    hf, Wf = f64(h), f64(W)
    dh, dW = O.backward(h, W, t, 3, g_l, g_e, temperature=0.7)
    eps = 1e-6
    for mat, grad, name in ((hf, dh, "dh"), (Wf, dW, "dW")):
        num = np.zeros_like(mat)
        for idx in np.ndindex(mat.shape):
            keep = mat[idx]
            mat[idx] = keep + eps
            up = O.loss(hf, Wf, t, g_l, g_e, temperature=0.7)
            mat[idx] = keep - eps
            dn = O.loss(hf, Wf, t, g_l, g_e, temperature=0.7)
            mat[idx] = keep
            num[idx] = (up - dn) / (2 * eps)
        _close(grad, num, 1e-7, 1e-8, what=f"T=0.7 {name} vs central differences")


def pin_temperature_limit():
    """T -> infinity flattens the distribution: logp -> -ln V, entropy -> ln V,
    lse - ln V -> mean(z) / T; the gradients vanish like 1 / T."""
    h, W, t, g_l, g_e = _rand_case(13, 6, 8, 11, w_std=0.5)
    V = W.shape[0]
    T = 1e9
    r = O.forward_backward(h, W, t, 4, g_l, g_e, temperature=T)
    z = f64(h) @ f64(W).T
    _close(r["logp"], np.full(6, -math.log(V)), 0.0, 1e-8, what="T->inf logp")
    _close(r["entropy"], np.full(6, math.log(V)), 0.0, 1e-8, what="T->inf entropy")
    _close(r["lse"] - math.log(V), z.mean(axis=1) / T, 1e-6, 1e-15, what="T->inf lse - ln V")
    # dh_i -> (g_l (W[t_i] - mean W)) / T at uniform p (the entropy term vanishes)
    Wf = f64(W)
    ref_dh = g_l[:, None] * (Wf[t] - Wf.mean(axis=0)[None, :]) / T
    _close(r["dh"], ref_dh, 1e-6, 1e-20, what="T->inf dh")


# --- non-finite logits (unmasked rows) ---------------------------------------------
# tunix #2913 checks its fused scoring against the textbook log-softmax and
# entropy on logits with inf, -inf and NaN entries and a row of no finite
# logit. Reading: IEEE evaluation of the definitions, the log-sum-exp shifted
# by the row max when it is finite and by 0 otherwise.

_BF16_POS_INF, _BF16_NEG_INF, _BF16_NAN = 0x7F80, 0xFF80, 0x7FC0


def _special_case(seed=21, N=6, H=5, V=9):
    rng = np.random.default_rng(seed)
    h = bf16(np.abs(rng.standard_normal((N, H))) + 0.25)    # h[:, 0] > 0: inf * h0 keeps its sign
    W = bf16(rng.standard_normal((V, H)) * 0.5)
    t = rng.integers(0, V, size=N).astype(np.int32)
    return h, W, t


def _row_only(W, v, first):
    W = W.copy()
    W[v] = 0
    W[v, 0] = first
    return W


def pin_nonfinite_logits():
    """Closed forms of the non-finite cases: a -inf entry drops out (equal to
    the row without that vocabulary entry) and makes the entropy NaN; a -inf
    target gives logp = -inf; +inf gives lse = +inf and logp = -inf (NaN at a
    +inf target); NaN makes everything NaN; a row of no finite logit has
    lse = -inf and NaN logp and entropy. Masked tokens stay exactly 0."""
    h, W, t = _special_case()
    N, V = h.shape[0], W.shape[0]
    v = 4
    t[:] = np.where(t == v, 0, t)
    t[1] = v                       # token 1 targets the special row
    t[5] = -1                      # token 5 is masked

    def run(Wb, tb=t, hb=h):
        return O.forward(hb, Wb, tb, 4)

    keep = np.array([i for i in range(V) if i != v])
    t_red = np.where(t > v, t - 1, t)

    # -inf entry: drops out of lse; -inf target -> logp -inf; entropy NaN
    lp, en, ls = run(_row_only(W, v, _BF16_NEG_INF))
    rlp, ren, rls = O.forward(h, W[keep], np.where(t == v, 0, t_red), 4)
    others = np.array([0, 2, 3, 4])
    _close(ls[others], rls[others], 1e-14, 1e-15, what="-inf entry: lse without it")
    _close(lp[others], rlp[others], 1e-14, 1e-15, what="-inf entry: logp without it")
    _close(ls[1], rls[1], 1e-14, 1e-15, what="-inf target: lse without it")
    assert lp[1] == -np.inf, "a -inf target logit gives logp = -inf"
    assert np.all(np.isnan(en[[0, 1, 2, 3, 4]])), "entropy of a row with a -inf entry is NaN (0 * -inf)"
    assert lp[5] == en[5] == ls[5] == 0.0

    # +inf entry: lse = +inf, logp = -inf (finite target) / NaN (the +inf target), entropy NaN
    lp, en, ls = run(_row_only(W, v, _BF16_POS_INF))
    assert np.all(ls[[0, 1, 2, 3, 4]] == np.inf), "+inf entry: lse = +inf"
    assert np.all(lp[others] == -np.inf) and np.isnan(lp[1]), "+inf entry: logp = -inf, NaN at the target"
    assert np.all(np.isnan(en[[0, 1, 2, 3, 4]]))
    assert lp[5] == en[5] == ls[5] == 0.0

    # NaN entry: everything NaN
    lp, en, ls = run(_row_only(W, v, _BF16_NAN))
    for name, a in (("logp", lp), ("entropy", en), ("lse", ls)):
        assert np.all(np.isnan(a[[0, 1, 2, 3, 4]])), f"NaN entry: {name} NaN"
        assert a[5] == 0.0

    # a row of no finite logit: token 2's hidden is [+inf, 0, ...] and W[:, 0] < 0
    W2 = W.copy()
    W2[:, 0] = bf16(-(np.abs(f64(W[:, 0])) + 0.125))
    h2 = h.copy()
    h2[2] = 0
    h2[2, 0] = _BF16_POS_INF
    lp, en, ls = run(W2, hb=h2)
    assert ls[2] == -np.inf and np.isnan(lp[2]) and np.isnan(en[2]), "no finite logit: lse -inf, NaN logp/entropy"
    rlp, ren, rls = run(W2)
    fine = np.array([0, 1, 3, 4])
    for a, r, name in ((lp, rlp, "logp"), (en, ren, "entropy"), (ls, rls, "lse")):
        _close(a[fine], r[fine], 0.0, 0.0, what=f"other tokens unaffected ({name})")



def pin_nonfinite_gradients():
    """Gradients at non-finite logits. Readings: the entropy term is formed
    only for tokens with a nonzero entropy cotangent (the one-pass g_l
    (onehot - p) form of a loss that stops the entropy's gradient), and an
    entry of probability 0 gets no probability term. Closed forms:
      * -inf entry v, log-prob cotangents only: the cotangent is g_l at a -inf
        target and 0 elsewhere in column v, so dW[v] = sum of g_l h over the
        tokens that target v (0 when none does); every other dW row and the
        columns of dh where W[v] is finite equal the gradients of the
        vocabulary without v; dh's column where W[v] = -inf is 0 * -inf = NaN
        for the other tokens and -sign(g_l) inf for the tokens targeting v;
      * the same with entropy cotangents: the entropy is NaN, so every entry
        of positive probability gets a NaN cotangent, while column v (p = 0)
        keeps the closed form above;
      * +inf entry, log-prob cotangents only: lse = +inf, every finite
        logit's probability is 0, so dW[u] = sum of g_l h over the tokens
        that target u for u != v, dW[v] is NaN and every unmasked dh row NaN;
      * NaN entry: every unmasked dh row and every dW entry is NaN.
    Masked rows stay 0 in every case."""
    h, W, t = _special_case(seed=22, N=7, H=5, V=9)
    N, V = h.shape[0], W.shape[0]
    rng = np.random.default_rng(5)
    g_l = rng.standard_normal(N) + np.where(rng.standard_normal(N) > 0, 0.5, -0.5)   # no zero
    g_e = rng.standard_normal(N) * 0.3 + 0.05
    v = 4
    t[:] = np.where(t == v, 0, t)
    t[6] = -1                          # token 6 is masked
    hf = f64(h)
    keep = np.array([i for i in range(V) if i != v])
    t_red = np.where(t > v, t - 1, t)
    live = np.array([i for i in range(N) if t[i] >= 0])

    # -inf entry, no token targets it, log-prob cotangents only
    Wm = _row_only(W, v, _BF16_NEG_INF)
    dh, dW = O.backward(h, Wm, t, 3, g_l, None)
    rdh, rdW = O.backward(h, W[keep], t_red, 3, g_l, None)
    assert np.all(dW[v] == 0.0), "-inf entry: its dW row is 0 when no token targets it"
    _close(dW[keep], rdW, 1e-13, 1e-15, what="-inf entry: other dW rows = vocabulary without it")
    _close(dh[:, 1:], rdh[:, 1:], 1e-13, 1e-15, what="-inf entry: dh columns of finite W[v]")
    assert np.all(np.isnan(dh[live, 0])), "-inf entry: 0 * -inf in the dh product"
    assert np.all(dh[6] == 0.0), "masked dh row"
    # with entropy cotangents (all nonzero): NaN entropy reaches every entry of positive probability
    dh, dW = O.backward(h, Wm, t, 3, g_l, g_e)
    assert np.all(dW[v] == 0.0), "-inf entry: p = 0 column carries no probability term"
    assert np.all(np.isnan(dW[keep])), "entropy cotangent on a NaN entropy"
    assert np.all(np.isnan(dh[live])) and np.all(dh[6] == 0.0)
    # a token that targets the -inf entry
    t2 = t.copy()
    t2[1] = v
    dh, dW = O.backward(h, Wm, t2, 3, g_l, None)
    _close(dW[v], g_l[1] * hf[1], 1e-15, 0.0, what="-inf target: dW[v] = g_l h")
    assert dh[1, 0] == -np.sign(g_l[1]) * np.inf, "-inf target: g_l * -inf in the dh product"
    assert np.all(np.isfinite(dh[:, 1:])) and np.all(np.isfinite(dW)), "finite elsewhere"

    # +inf entry, log-prob cotangents only
    Wp = _row_only(W, v, _BF16_POS_INF)
    dh, dW = O.backward(h, Wp, t, 3, g_l, None)
    want = np.zeros((V, h.shape[1]))
    for i in live:
        want[t[i]] += g_l[i] * hf[i]
    _close(dW[keep], want[keep], 1e-15, 0.0, what="+inf entry: finite entries have p = 0")
    assert np.all(np.isnan(dW[v])) and np.all(np.isnan(dh[live])) and np.all(dh[6] == 0.0)

    # NaN entry
    dh, dW = O.backward(h, _row_only(W, v, _BF16_NAN), t, 3, g_l, g_e)
    assert np.all(np.isnan(dW)) and np.all(np.isnan(dh[live])) and np.all(dh[6] == 0.0)


def pin_bruteforce_random():
    """The 50-digit brute force on random tiny cases: shapes from one token,
    one hidden unit and one vocabulary row up, every chunk size from 1 to past
    N, masked ids -1 and V, temperatures below and above 1, and W scales up
    to 2 (logits in the tens, peaked softmaxes); forward values and both
    gradients."""
    rng = np.random.default_rng(2024)
    temps = ("1", "0.5", "0.7", "2")
    for case in range(8):
        N = int(rng.integers(1, 5))
        H = int(rng.integers(1, 6))
        V = int(rng.integers(1, 8))
        C = int(rng.integers(1, N + 2))
        T = temps[case % len(temps)]
        w_std = float(rng.uniform(0.3, 2.0))
        h = bf16(rng.standard_normal((N, H)))
        W = bf16(rng.standard_normal((V, H)) * w_std)
        t = rng.integers(0, V, size=N).astype(np.int32)
        if N > 1:
            t[int(rng.integers(0, N))] = (-1, V)[case % 2]
        g_l = rng.standard_normal(N)
        g_e = rng.standard_normal(N) * 0.3
        what = f"random case {case} (N={N} H={H} V={V} C={C} T={T})"
        logp, ent, lse = O.forward(h, W, t, C, temperature=float(T))
        for i, (lp, en, ls) in enumerate(B.forward(h.tolist(), W.tolist(), t.tolist(), temperature=T)):
            _close(logp[i], float(lp), 1e-12, 1e-14, what=f"{what} logp[{i}]")
            _close(ent[i], float(en), 1e-12, 1e-14, what=f"{what} entropy[{i}]")
            _close(lse[i], float(ls), 1e-12, 1e-14, what=f"{what} lse[{i}]")
        dh, dW = O.backward(h, W, t, C, g_l, g_e, temperature=float(T))
        rdh, rdW = B.gradients(h.tolist(), W.tolist(), t.tolist(), g_l, g_e, temperature=T)
        rdh = np.array([[float(x) for x in row] for row in rdh])
        rdW = np.array([[float(x) for x in row] for row in rdW])
        _close(dh, rdh, 1e-10, 1e-12 * max(1e-300, np.abs(rdh).max()), what=f"{what} dh")
        _close(dW, rdW, 1e-10, 1e-12 * max(1e-300, np.abs(rdW).max()), what=f"{what} dW")


ALL_PINS = [
    pin_W_zero,
    pin_h_zero,
    pin_V1,
    pin_V2,
    pin_bruteforce_forward,
    pin_bruteforce_gradients,
    pin_bruteforce_random,
    pin_fd_gradients,
    pin_normalisation,
    pin_shift_invariance,
    pin_masking,
    pin_chunk_invariance,
    pin_subset_evaluation,
    pin_temperature_power_of_two,
    pin_temperature_bruteforce,
    pin_temperature_fd,
    pin_temperature_limit,
    pin_nonfinite_logits,
    pin_nonfinite_gradients,
]
