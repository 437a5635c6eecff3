"""Non-finite logits in unmasked rows on the GPU against the fp64 oracle
(google/tunix pull request #2913 checks its fused scoring on logits with inf,
-inf and NaN entries and a row of no finite logit). Reading: IEEE evaluation
of the definitions with the log-sum-exp shifted by the row max when finite
and by 0 otherwise; so NaN, +inf and -inf must land exactly where the oracle
puts them and finite values must meet the usual bar."""
import numpy as np
import pytest

import oracle.lmhead_oracle as O
from gpu_common import ATOL, RTOL, log, run_head
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
