"""Plausible mistakes planted in the fp64 oracle (on the CPU) must each be
caught by at least one pin. This is what makes the pins trustworthy: a pin set
that a sign flip or a dropped term slips through pins nothing.

The mistake list follows the kinds of broken copies google/tunix pull request
#2913 reports catching in its fused-head tests (cotangent sign flipped, max
dropped from the log-probs, max and exp-sum swapped, entropy sign flipped,
vocabulary bound off by one, wrap of negative ids, isfinite mask dropped),
plus transposed operands and dropped terms, and the tempered head's
mistakes (temperature ignored or multiplied, the backward's division by the
temperature dropped), and the non-finite cotangent's readings broken (0 times
a NaN entropy or a -inf log-probability leaking in, the entropy term formed
without its cotangent, a probability term kept where the probability is 0)."""
import numpy as np
import pytest

import oracle.lmhead_oracle as O
from oracle_pins import ALL_PINS


def _m_cotangent_sign(z, lse, p, ent, t, g_l, g_e):
    return -_orig["_cotangent"](z, lse, p, ent, t, g_l, g_e)


def _m_entropy_term_sign(z, lse, p, ent, t, g_l, g_e):
    dz = -g_l[:, None] * p + g_e[:, None] * p * ((z - lse[:, None]) + ent[:, None])
    dz[np.arange(z.shape[0]), t] += g_l
    return dz


def _m_entropy_term_dropped_H(z, lse, p, ent, t, g_l, g_e):
    dz = -g_l[:, None] * p - g_e[:, None] * p * (z - lse[:, None])
    dz[np.arange(z.shape[0]), t] += g_l
    return dz


def _m_onehot_off_by_one(z, lse, p, ent, t, g_l, g_e):
    dz = -g_l[:, None] * p - g_e[:, None] * p * ((z - lse[:, None]) + ent[:, None])
    dz[np.arange(z.shape[0]), (t + 1) % z.shape[1]] += g_l
    return dz


def _m_cotangent_swapped_g(z, lse, p, ent, t, g_l, g_e):
    return _orig["_cotangent"](z, lse, p, ent, t, g_e, g_l)


def _m_lse_dropped_max(z):
    m = np.max(z, axis=1, keepdims=True)
    return np.log(np.sum(np.exp(z - m), axis=1))


def _m_lse_max_and_sum_swapped(z):
    m = np.max(z, axis=1, keepdims=True)
    s = np.sum(np.exp(z - m), axis=1, keepdims=True)
    return (s + np.log(m * 0 + np.abs(m) + 1e-300))[:, 0]


def _m_entropy_sign(z, lse, p):
    return np.sum(p * (z - lse[:, None]), axis=1)


def _m_entropy_no_lse(z, lse, p):
    return -np.sum(p * z, axis=1)


def _m_valid_bound_off_by_one(targets, V):
    t = np.asarray(targets, dtype=np.int64)
    return (t >= 0) & (t <= V - 2)


def _m_valid_wraps_negative(targets, V):
    t = np.asarray(targets, dtype=np.int64)
    return t < V


def _m_target_logit_first_row(z, t):
    return z[np.arange(z.shape[0]), np.zeros_like(t)]


def _m_logits_transposed_scale(h_rows, W):
    return h_rows @ W.T * 0.5


def _m_probs_unnormalised(z, lse):
    return np.exp(z - np.max(z, axis=1, keepdims=True))


def _m_temperature_ignored(z, temperature):
    return z


def _m_temperature_multiplied(z, temperature):
    return z * temperature


def _m_backward_temperature_division_dropped(dz, temperature):
    return dz


def _m_lse_shift_always_max(z):
    m = np.max(z, axis=1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        return (m + np.log(np.sum(np.exp(z - m), axis=1, keepdims=True)))[:, 0]


def _m_entropy_zero_times_log_zero(z, lse, p):
    with np.errstate(invalid="ignore"):
        return -np.sum(np.where(p > 0, p * (z - lse[:, None]), 0.0), axis=1)



def _m_cotangent_plain_ieee(z, lse, p, ent, t, g_l, g_e):
    # no selects: 0 * NaN (a NaN entropy under a zero entropy cotangent) and
    # 0 * -inf (log p at p = 0) leak into the cotangent
    with np.errstate(invalid="ignore"):
        dz = -g_l[:, None] * p - g_e[:, None] * p * ((z - lse[:, None]) + ent[:, None])
    dz[np.arange(z.shape[0]), t] += g_l
    return dz


def _m_entropy_term_without_cotangent(z, lse, p, ent, t, g_l, g_e):
    with np.errstate(invalid="ignore", over="ignore"):
        bracket = g_l[:, None] + g_e[:, None] * ((z - lse[:, None]) + ent[:, None])
        dz = -np.where(p == 0.0, 0.0, p * bracket)
    dz[np.arange(z.shape[0]), t] += g_l
    return dz


def _m_prob_term_at_zero_probability(z, lse, p, ent, t, g_l, g_e):
    with np.errstate(invalid="ignore", over="ignore"):
        ent_term = np.where(g_e[:, None] != 0.0, g_e[:, None] * ((z - lse[:, None]) + ent[:, None]), 0.0)
        dz = -p * (g_l[:, None] + ent_term)
    dz[np.arange(z.shape[0]), t] += g_l
    return dz

_orig = {}

MUTANTS = {
    "cotangent_sign": ("_cotangent", _m_cotangent_sign),
    "entropy_term_sign": ("_cotangent", _m_entropy_term_sign),
    "entropy_term_missing_H": ("_cotangent", _m_entropy_term_dropped_H),
    "onehot_off_by_one": ("_cotangent", _m_onehot_off_by_one),
    "cotangents_swapped": ("_cotangent", _m_cotangent_swapped_g),
    "lse_max_dropped": ("_log_sum_exp", _m_lse_dropped_max),
    "lse_max_expsum_swapped": ("_log_sum_exp", _m_lse_max_and_sum_swapped),
    "entropy_sign": ("_entropy", _m_entropy_sign),
    "entropy_without_lse": ("_entropy", _m_entropy_no_lse),
    "vocab_bound_off_by_one": ("valid_targets", _m_valid_bound_off_by_one),
    "negative_ids_wrap": ("valid_targets", _m_valid_wraps_negative),
    "target_logit_wrong_index": ("_target_logit", _m_target_logit_first_row),
    "logits_scaled": ("_logits", _m_logits_transposed_scale),
    "probs_unnormalised": ("_probs", _m_probs_unnormalised),
    "temperature_ignored": ("_temper", _m_temperature_ignored),
    "temperature_multiplied": ("_temper", _m_temperature_multiplied),
    "backward_temperature_division_dropped": ("_raw_cotangent", _m_backward_temperature_division_dropped),
    "lse_shift_by_nonfinite_max": ("_log_sum_exp", _m_lse_shift_always_max),
    "entropy_zero_log_zero_convention": ("_entropy", _m_entropy_zero_times_log_zero),
    "cotangent_zero_times_nonfinite": ("_cotangent", _m_cotangent_plain_ieee),
    "entropy_term_without_its_cotangent": ("_cotangent", _m_entropy_term_without_cotangent),
    "probability_term_at_zero_probability": ("_cotangent", _m_prob_term_at_zero_probability),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    _orig[attr] = getattr(O, attr)
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            pin()
        except (AssertionError, IndexError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
            break
    assert caught, f"mutant {name} passed every pin"
