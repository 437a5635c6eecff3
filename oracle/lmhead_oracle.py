"""fp64 CPU oracle of the chunked LM-head log-prob and entropy head.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or run anything under
``oracle/``. The product path (``cross_entropy_amd``) never calls it, and
this module imports nothing from the product path: the two share no kernels,
headers, helpers, tables or pre/post-processing.

What it computes is the plain definition, written out in float64 numpy, with
the full logits row of every token materialised:

For each chunk of ``chunk_size`` flattened tokens, in order, and each token i
of the chunk with hidden row h_i and target id t_i:

1. validity: t_i is a real target iff 0 <= t_i < V; any other id (the
   padding id -1 included) masks the token. Masked tokens have
   logp = entropy = lse = 0 and contribute nothing to dh or dW.
   [google/tunix pull request #2913, review of ``_target_hit``: the hit mask
   is paired with ``(ids >= 0) & (ids < vocab)``.]
2. logits z = W h_i over the whole vocabulary (a row of V values).
   [SkyRL issue "[tx] support long sequence", "4. Chunked LM Head": the loss
   is computed chunk by chunk instead of on the full logits tensor.]
3. lse = m + log(sum_v exp(z_v - m)) with m = max_v z_v; p = exp(z - lse).
4. logp = z[t_i] - lse  (the target logit minus the log of the exp-sum plus
   the max) and entropy = -sum_v p_v (z_v - lse) (natural log, nats).
   [tunix #2913, "How the fused log-prob head works": each token's log-prob
   is the target logit minus (log exp-sum + max); the entropy comes from the
   same exponentials. Its "local" head defines the values with
   selective_log_softmax and compute_entropy_from_logits.]
5. backward of L = sum_i g_logp_i * logp_i + g_ent_i * entropy_i:
   dz = g_logp (onehot(t) - p) - g_ent p (log p + entropy), log p = z - lse;
   dh_i = W^T dz; dW += dz h_i^T.

Temperature T > 0 (default 1): the head scores the tempered logits z / T,
so every statistic above is that of softmax(z / T), and the backward divides
the tempered logits' cotangent by T before both gradient matmuls (chain rule
through z / T).
   [tunix #2913 runs its head tests at temperatures 1 and 0.7 and lists
   "the backward's temperature division dropped" among the broken copies
   its tests must catch.]
   [tunix #2913: the logits' cotangent in one elementwise pass over the
   recomputed logits when only the log-probs carry a cotangent; a loss that
   differentiates the entropy adds the entropy term; both gradient matmuls
   read that one cotangent.]

Non-finite logits (unmasked rows; they arise only from non-finite W or
hidden values). tunix #2913 checks its fused scoring against the textbook
log-softmax and entropy on logits with inf, -inf and NaN entries and on a row
of no finite logit. The reading taken here is IEEE evaluation of the
definitions above, with the log-sum-exp shifted by the row max when that max
is finite and by 0 otherwise:
  * -inf entries have exp = 0 and drop out of lse; a -inf target gives
    logp = -inf; the entropy's p * (z - lse) is 0 * -inf = NaN;
  * a +inf entry (and no NaN) gives lse = +inf, logp = -inf for a finite
    target and NaN for a +inf target, entropy NaN;
  * a NaN entry makes lse, logp and entropy NaN;
  * a row of no finite logit (all -inf) has lse = -inf, logp = entropy = NaN.
Gradients follow the same IEEE arithmetic, with two readings in the
cotangent (step 5): the entropy term is formed only for tokens with a nonzero
entropy cotangent, and an entry of probability 0 gets no probability term.
So with only log-prob cotangents a -inf entry's cotangent is g_l at a -inf
target and 0 elsewhere, and the rest of the row is that of the vocabulary
without it (the products of the two gradient matmuls stay IEEE: a cotangent
of 0 times the -inf table entry is NaN in dh). Masked rows stay exactly 0.

Readings taken where the pages leave a step open: chunk_size counts flattened
tokens, the last chunk may be partial (tunix #2913 tests "chunks that do not
divide the local sequence and one chunk for all of it"); masked lse is 0;
entropy is in nats; there is no cotangent on lse; a missing cotangent is 0.

Every value here is pinned by ``tests/test_oracle.py`` against closed forms,
invariants, 50-digit brute force (``oracle/bruteforce.py``) and central
finite differences, not against this module itself.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

__all__ = [
    "widen_bf16",
    "valid_targets",
    "chunk_ranges",
    "forward",
    "backward",
    "forward_backward",
    "loss",
]


def widen_bf16(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (a bf16 value is the top
    16 bits of the float32 with the same value)."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("bf16 inputs are passed as uint16 bit patterns")
    f32 = (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f32.astype(np.float64)


def valid_targets(targets: np.ndarray, V: int) -> np.ndarray:
    """Step 1: a target id is real iff 0 <= id < V."""
    t = np.asarray(targets, dtype=np.int64)
    return (t >= 0) & (t < V)


def chunk_ranges(N: int, chunk_size: int):
    """The chunk loop: ceil(N / chunk_size) chunks of flattened tokens, the
    last one partial when chunk_size does not divide N."""
    if chunk_size <= 0:
        raise ValueError("chunk_size must be positive")
    return [(s, min(N, s + chunk_size)) for s in range(0, N, chunk_size)]


def _logits(h_rows: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Step 2: z = h W^T, one full row of V logits per token."""
    return h_rows @ W.T


def _temper(z: np.ndarray, temperature: float) -> np.ndarray:
    """The tempered logits z / T that the head scores."""
    return z / temperature


def _raw_cotangent(dz: np.ndarray, temperature: float) -> np.ndarray:
    """Chain rule through z / T: the untempered logits' cotangent is dz / T."""
    return dz / temperature


def _log_sum_exp(z: np.ndarray) -> np.ndarray:
    """Step 3: lse = m + log(sum exp(z - m)) per row, m the row max when it is
    finite and 0 otherwise (a row holding +inf, NaN or only -inf)."""
    m = np.max(z, axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        return (m + np.log(np.sum(np.exp(z - m), axis=1, keepdims=True)))[:, 0]


def _probs(z: np.ndarray, lse: np.ndarray) -> np.ndarray:
    """p = exp(z - lse) per row."""
    with np.errstate(invalid="ignore", over="ignore"):
        return np.exp(z - lse[:, None])


def _target_logit(z: np.ndarray, t: np.ndarray) -> np.ndarray:
    """z[t] per row (t already known to be valid)."""
    return z[np.arange(z.shape[0]), t]


def _entropy(z: np.ndarray, lse: np.ndarray, p: np.ndarray) -> np.ndarray:
    """Step 4: entropy = -sum_v p_v log p_v with log p = z - lse."""
    with np.errstate(invalid="ignore"):
        return -np.sum(p * (z - lse[:, None]), axis=1)


def _cotangent(z, lse, p, ent, t, g_l, g_e) -> np.ndarray:
    """Step 5: dz = g_l onehot(t) - p (g_l + g_e (log p + entropy)).

    Two readings settle what IEEE arithmetic alone leaves open where logits
    are non-finite (finite logits give the same values either way):
      * the entropy term is formed only for tokens whose entropy cotangent is
        nonzero: a token that carries only a log-prob cotangent takes the
        one-pass form g_l (onehot - p) (tunix #2913: the backward of a loss
        that stops the entropy's gradient), so a NaN entropy (a row with a
        -inf entry) never reaches its gradient;
      * an entry whose probability is exactly 0 (a -inf logit, or every
        finite logit of a row whose lse is +inf) gets no probability term,
        whatever the bracket holds: p (log p + H) -> 0 as p -> 0.
    """
    with np.errstate(invalid="ignore", over="ignore"):
        ent_term = np.where(g_e[:, None] != 0.0, g_e[:, None] * ((z - lse[:, None]) + ent[:, None]), 0.0)
        prob_term = np.where(p == 0.0, 0.0, p * (g_l[:, None] + ent_term))
    dz = -prob_term
    dz[np.arange(z.shape[0]), t] += g_l
    return dz


def _check_temperature(temperature):
    T = float(temperature)
    if not (np.isfinite(T) and T > 0.0):
        raise ValueError("temperature must be finite and > 0")
    return T


def _rows_stats(h_rows, W, t, temperature=1.0):
    with np.errstate(invalid="ignore", over="ignore"):
        z = _temper(_logits(h_rows, W), temperature)
    lse = _log_sum_exp(z)
    p = _probs(z, lse)
    with np.errstate(invalid="ignore"):
        logp = _target_logit(z, t) - lse
    ent = _entropy(z, lse, p)
    return z, lse, p, logp, ent


def _prepare(hidden_bits, W_bits, targets):
    h = widen_bf16(hidden_bits)
    W = widen_bf16(W_bits)
    if h.ndim != 2 or W.ndim != 2 or h.shape[1] != W.shape[1]:
        raise ValueError("hidden [N,H] and W [V,H] must share H")
    t = np.asarray(targets, dtype=np.int64).reshape(-1)
    if t.shape[0] != h.shape[0]:
        raise ValueError("targets must have N entries")
    return h, W, t


def _token_blocks(lo: int, hi: int, row_block: int):
    for s in range(lo, hi, row_block):
        yield s, min(hi, s + row_block)


def forward(hidden_bits, W_bits, targets, chunk_size: int, tokens: Optional[np.ndarray] = None,
            row_block: int = 256, temperature: float = 1.0):
    """Forward values (logp, entropy, lse), float64 arrays.

    ``tokens``: optional sorted index subset; then only those tokens are
    computed (each token needs only its own logits row) and the arrays have
    ``len(tokens)`` entries. ``row_block`` only sets how many tokens of a
    chunk are evaluated per numpy call; the values do not depend on it.
    """
    T = _check_temperature(temperature)
    h, W, t = _prepare(hidden_bits, W_bits, targets)
    N, V = h.shape[0], W.shape[0]
    ids = np.arange(N) if tokens is None else np.asarray(tokens, dtype=np.int64)
    valid = valid_targets(t, V)
    pos = {int(i): k for k, i in enumerate(ids)} if tokens is not None else None
    logp = np.zeros(ids.shape[0])
    ent = np.zeros(ids.shape[0])
    lse = np.zeros(ids.shape[0])
    for c0, c1 in chunk_ranges(N, chunk_size):
        sel = ids[(ids >= c0) & (ids < c1)]
        sel = sel[valid[sel]]
        for b0 in range(0, sel.shape[0], row_block):
            rows = sel[b0:b0 + row_block]
            _, l, _, lp, en = _rows_stats(h[rows], W, t[rows], T)
            out = rows if pos is None else np.array([pos[int(i)] for i in rows], dtype=np.int64)
            logp[out], ent[out], lse[out] = lp, en, l
    return logp, ent, lse


def backward(hidden_bits, W_bits, targets, chunk_size: int, g_logp=None, g_ent=None,
             tokens: Optional[np.ndarray] = None, row_block: int = 256, temperature: float = 1.0):
    """Gradients (dh, dW) of L = sum_i g_logp_i logp_i + g_ent_i entropy_i.

    ``g_logp`` / ``g_ent`` of None mean zero. dh is [N, H] (or
    [len(tokens), H] with ``tokens``), dW is [V, H], both float64. With
    ``tokens``, dW sums only those tokens' contributions: this equals the full
    dW exactly when every other token's cotangents are zero.
    Masked tokens give dh rows of 0 and nothing to dW, whatever their hidden
    row holds (they are never multiplied, only skipped)."""
    T = _check_temperature(temperature)
    h, W, t = _prepare(hidden_bits, W_bits, targets)
    N, H = h.shape
    V = W.shape[0]
    g_l = np.zeros(N) if g_logp is None else np.asarray(g_logp, dtype=np.float64).reshape(-1)
    g_e = np.zeros(N) if g_ent is None else np.asarray(g_ent, dtype=np.float64).reshape(-1)
    ids = np.arange(N) if tokens is None else np.asarray(tokens, dtype=np.int64)
    pos = {int(i): k for k, i in enumerate(ids)} if tokens is not None else None
    valid = valid_targets(t, V)
    dh = np.zeros((ids.shape[0], H))
    dW = np.zeros((V, H))
    for c0, c1 in chunk_ranges(N, chunk_size):
        sel = ids[(ids >= c0) & (ids < c1)]
        sel = sel[valid[sel]]
        for b0 in range(0, sel.shape[0], row_block):
            rows = sel[b0:b0 + row_block]
            z, l, p, _, en = _rows_stats(h[rows], W, t[rows], T)
            dz = _raw_cotangent(_cotangent(z, l, p, en, t[rows], g_l[rows], g_e[rows]), T)
            out = rows if pos is None else np.array([pos[int(i)] for i in rows], dtype=np.int64)
            with np.errstate(invalid="ignore", over="ignore"):
                dh[out] = dz @ W
                dW += dz.T @ h[rows]
    return dh, dW


def forward_backward(hidden_bits, W_bits, targets, chunk_size: int, g_logp=None, g_ent=None,
                     tokens: Optional[np.ndarray] = None, row_block: int = 256, temperature: float = 1.0):
    """Both passes; returns dict(logp, entropy, lse, dh, dW)."""
    logp, ent, lse = forward(hidden_bits, W_bits, targets, chunk_size, tokens, row_block, temperature)
    dh, dW = backward(hidden_bits, W_bits, targets, chunk_size, g_logp, g_ent, tokens, row_block, temperature)
    return {"logp": logp, "entropy": ent, "lse": lse, "dh": dh, "dW": dW}


def loss(hidden_f64: np.ndarray, W_f64: np.ndarray, targets, g_logp, g_ent, temperature: float = 1.0) -> float:
    """L = sum_i g_logp_i logp_i + g_ent_i entropy_i on float64 inputs (for
    finite-difference checks of ``backward``); masked tokens add nothing."""
    T = _check_temperature(temperature)
    t = np.asarray(targets, dtype=np.int64)
    V = W_f64.shape[0]
    valid = valid_targets(t, V)
    rows = np.flatnonzero(valid)
    if rows.size == 0:
        return 0.0
    _, _, _, lp, en = _rows_stats(hidden_f64[rows], W_f64, t[rows], T)
    g_l = np.asarray(g_logp, dtype=np.float64)[rows]
    g_e = np.asarray(g_ent, dtype=np.float64)[rows]
    return float(np.sum(g_l * lp) + np.sum(g_e * en))
