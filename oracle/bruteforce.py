"""50-digit brute force of the LM-head log-prob / entropy head, tiny shapes.

TEST INFRASTRUCTURE ONLY (same rule as ``oracle/lmhead_oracle.py``). It
shares no code with the fp64 oracle: it works in Python ``decimal`` with the
unshifted textbook definitions and pins that oracle in ``tests/``.

* log p(t) = log( exp(z_t) / sum_v exp(z_v) )      (no max subtraction)
* entropy  = -sum_v p_v log p_v,  p_v = exp(z_v) / sum_u exp(z_u)
* lse      = log sum_v exp(z_v)
* gradients of L = sum_i g_logp_i log p_i(t_i) + g_ent_i entropy_i by central
  differences at step 1e-20 in 60-digit arithmetic (error ~1e-38, far below
  float64 resolution).

Temperature T (default 1) divides every logit: z_v = (h . W_v) / T, with T
given as a decimal string and held exactly.

Inputs are exact: bf16 values are dyadic rationals, which Decimal holds
exactly. Only for N <= 4, H <= 8, V <= 16 or so: every derivative costs two
full evaluations.
"""
from __future__ import annotations

from decimal import Decimal, localcontext

__all__ = ["bf16_bits_to_decimal", "forward", "loss", "gradients"]

_PREC = 60


def bf16_bits_to_decimal(bits: int) -> Decimal:
    """Exact value of one bfloat16 bit pattern (finite values only)."""
    bits = int(bits) & 0xFFFF
    sign = -1 if bits & 0x8000 else 1
    exp = (bits >> 7) & 0xFF
    man = bits & 0x7F
    if exp == 0xFF:
        raise ValueError("non-finite bf16 value")
    with localcontext() as ctx:
        ctx.prec = _PREC
        if exp == 0:
            val = Decimal(man) * (Decimal(2) ** -133)          # subnormal: man * 2^-126 / 2^7
        else:
            val = (Decimal(128 + man)) * (Decimal(2) ** (exp - 127 - 7))
        return sign * val


def _matrix(bits_rows):
    return [[bf16_bits_to_decimal(b) for b in row] for row in bits_rows]


def _token(h_row, W, t, T=Decimal(1)):
    """(logp, entropy, lse) of one token from Decimal rows."""
    V = len(W)
    z = [sum(a * b for a, b in zip(h_row, W[v])) / T for v in range(V)]
    ez = [x.exp() for x in z]
    s = sum(ez)
    p = [e / s for e in ez]
    logp = (ez[t] / s).ln()
    ent = -sum(pv * pv.ln() for pv in p if pv != 0)
    lse = s.ln()
    return logp, ent, lse


def forward(hidden_bits, W_bits, targets, temperature: str = "1"):
    """Per-token (logp, entropy, lse) as Decimals; masked tokens give zeros."""
    with localcontext() as ctx:
        ctx.prec = _PREC
        T = Decimal(temperature)
        h = _matrix(hidden_bits)
        W = _matrix(W_bits)
        V = len(W)
        out = []
        for i, t in enumerate(targets):
            t = int(t)
            if 0 <= t < V:
                out.append(_token(h[i], W, t, T))
            else:
                out.append((Decimal(0), Decimal(0), Decimal(0)))
        return out


def loss(h, W, targets, g_logp, g_ent, T=Decimal(1)):
    """L on Decimal matrices (masked tokens add nothing)."""
    V = len(W)
    total = Decimal(0)
    for i, t in enumerate(targets):
        t = int(t)
        if not (0 <= t < V):
            continue
        logp, ent, _ = _token(h[i], W, t, T)
        total += Decimal(repr(float(g_logp[i]))) * logp + Decimal(repr(float(g_ent[i]))) * ent
    return total


def gradients(hidden_bits, W_bits, targets, g_logp, g_ent, step: str = "1e-20", temperature: str = "1"):
    """(dh, dW) as nested lists of Decimals by central differences of L."""
    with localcontext() as ctx:
        ctx.prec = _PREC
        T = Decimal(temperature)
        h = _matrix(hidden_bits)
        W = _matrix(W_bits)
        d = Decimal(step)

        def central(mat, r, c):
            keep = mat[r][c]
            mat[r][c] = keep + d
            up = loss(h, W, targets, g_logp, g_ent, T)
            mat[r][c] = keep - d
            dn = loss(h, W, targets, g_logp, g_ent, T)
            mat[r][c] = keep
            return (up - dn) / (2 * d)

        dh = [[central(h, r, c) for c in range(len(h[0]))] for r in range(len(h))]
        dW = [[central(W, r, c) for c in range(len(W[0]))] for r in range(len(W))]
        return dh, dW
