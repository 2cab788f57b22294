"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in the oracle (a dropped term, a wrong sign,
weight, index, orientation, bit order, tie rule or rounding), in this
process only, through pytest's monkeypatch, and runs the pins that cover
the function: at least one of them must fail.  A pin set that passed with
the mistake in place would not tell the oracle from its mutant.
"""
import math

import numpy as np
import pytest

from oracle import sm_oracle as O
from tests import test_oracle_pins as P


# ------------------------------------------------------------------ planted mistakes

def ema_weights_swapped(m_prev, g, beta):
    return (1.0 - beta) * np.asarray(m_prev, np.float64) + beta * np.asarray(g, np.float64)


def lion_interp_no_gradient(m_prev, g, beta1):
    return beta1 * np.asarray(m_prev, np.float64) + 0.0 * np.asarray(g, np.float64)


def lion_momentum_heavy_ball(m_prev, g, beta2):
    return beta2 * np.asarray(m_prev, np.float64) + np.asarray(g, np.float64)


def normalize_by_max(y, eps):
    y = np.asarray(y, np.float64)
    return y / (np.max(np.abs(y)) + eps)


def ns_sign_of_b_flipped(x, p):
    x = np.asarray(x, np.float64)
    for _ in range(p.iters):
        a_mat = x @ x.T
        b_mat = -p.b * a_mat
        if p.c != 0.0:
            b_mat = b_mat + p.c * (a_mat @ a_mat)
        x = p.a * x + b_mat @ x
    return x


def ns_quintic_term_dropped(x, p):
    x = np.asarray(x, np.float64)
    for _ in range(p.iters):
        x = p.a * x + p.b * (x @ x.T) @ x
    return x


def ns_one_iteration_short(x, p):
    x = np.asarray(x, np.float64)
    for _ in range(max(p.iters - 1, 0)):
        a_mat = x @ x.T
        b_mat = p.b * a_mat
        if p.c != 0.0:
            b_mat = b_mat + p.c * (a_mat @ a_mat)
        x = p.a * x + b_mat @ x
    return x


def gram_one_sided_update(x, p):
    x = np.asarray(x, np.float64)
    r = x.shape[0]
    eye = np.eye(r)
    g = x @ x.T
    q = eye.copy()
    for _ in range(p.iters):
        pk = p.a * eye + p.b * g
        if p.c != 0.0:
            pk = pk + p.c * (g @ g)
        q = pk @ q
        g = pk @ g            # missing the right-hand factor
    return q @ x, q


def residual_over_r(d):
    d = np.asarray(d, np.float64)
    r = d.shape[0]
    e = d @ d.T - np.eye(r)
    return math.sqrt(float(np.sum(e * e))) / r


def accept_strict(err, gamma):
    return bool(err < gamma)


def sign_nonpositive(x):
    return np.asarray(x) <= 0


def pack_msb_first(neg):
    neg = np.asarray(neg, dtype=bool).reshape(-1)
    n = neg.size
    nwords = (n + 63) // 64
    padded = np.zeros(nwords * 64, dtype=np.uint64)
    padded[:n] = neg.astype(np.uint64)
    weights = np.uint64(1) << np.arange(63, -1, -1, dtype=np.uint64)
    return (padded.reshape(nwords, 64) * weights).sum(axis=1, dtype=np.uint64)


def vote_ties_positive(bits_per_worker, count):
    m_workers = len(bits_per_worker)
    n_neg = np.zeros(count, dtype=np.int64)
    for words in bits_per_worker:
        n_neg += O.unpack_bits(words, count).astype(np.int64)
    s = m_workers - 2 * n_neg
    return np.where(s >= 0, 1, -1).astype(np.int8)


def update_vote_wrong_sign(w_values, v, lr, wdtype):
    w32 = np.asarray(w_values, dtype=np.float64).astype(np.float32)
    out32 = (w32 + np.float32(lr) * np.asarray(v).astype(np.float32)).astype(np.float32)
    if wdtype == O.F32:
        return out32.astype(np.float64)
    return O.f32_from_bf16_bits(O.bf16_bits_from_f32(out32)).astype(np.float64)


def update_vote_bf16_truncated(w_values, v, lr, wdtype):
    w32 = np.asarray(w_values, dtype=np.float64).astype(np.float32)
    out32 = (w32 - np.float32(lr) * np.asarray(v).astype(np.float32)).astype(np.float32)
    if wdtype == O.F32:
        return out32.astype(np.float64)
    bits = (out32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)   # no rounding
    return O.f32_from_bf16_bits(bits).astype(np.float64)


def sign_int8_zero_is_zero(x):
    return np.sign(np.nan_to_num(np.asarray(x, np.float64).reshape(-1))).astype(np.int8)


def vote_int8_ties_positive(signs_per_worker, count):
    total = np.zeros(count, dtype=np.int64)
    for sv in signs_per_worker:
        total += np.asarray(sv, dtype=np.int64).reshape(-1)[:count]
    return np.where(total >= 0, 1, -1).astype(np.int8)


def muon_phase_shifted(t, period):
    return period > 0 and t % period == 1 % period


def lion_sign_of_momentum_only(m_prev, g, beta1):
    return O.sign_negative(np.asarray(m_prev, np.float64))


def update_polar_one_rounding(w_values, d_values, lr, wdtype):
    w = np.asarray(w_values, dtype=np.float64).astype(np.float32).astype(np.float64)
    d = np.asarray(d_values, dtype=np.float64).astype(np.float32).astype(np.float64)
    out32 = (w - np.float64(np.float32(lr)) * d).astype(np.float32)   # lr * D not rounded
    if wdtype == O.F32:
        return out32.astype(np.float64)
    return O.f32_from_bf16_bits(O.bf16_bits_from_f32(out32)).astype(np.float64)


def power_without_normalising(e, v0, iters):
    e = np.asarray(e, np.float64)
    v = np.asarray(v0, np.float64).reshape(-1)
    with np.errstate(over="ignore", invalid="ignore"):
        for _ in range(iters):
            v = e.T @ (e @ v)
        y = e @ v
        return math.sqrt(float(y @ y))


def power_frobenius(e, v0, iters):
    return float(np.linalg.norm(np.asarray(e, np.float64)))


def orient_never_transposes(y):
    return np.asarray(y, np.float64).copy(), False


def vote_polar_unnormalised(v, p):
    return O.ns_polar(np.asarray(v, dtype=np.float64), p, normalize=False)


def unpack_reversed(words, count):
    words = np.asarray(words, dtype=np.uint64).reshape(-1)
    shifts = np.arange(63, -1, -1, dtype=np.uint64)
    bits = (words[:, None] >> shifts[None, :]) & np.uint64(1)
    return bits.reshape(-1)[:count].astype(bool)


# ------------------------------------------------------------------ cases

COEFS = [(1.5, -0.5, 0.0), (1.9, -0.7, 0.05), (1.2, -0.1, -0.08)]

CASES = [
    ("ema weights swapped", "ema", ema_weights_swapped,
     [lambda: P.test_p1_ema_constant_gradient_closed_form(0.9)]),
    ("Lion interpolation without the gradient", "lion_interp", lion_interp_no_gradient,
     [P.test_p1_lion_buffers_closed_form]),
    ("Lion buffer as heavy ball", "lion_momentum", lion_momentum_heavy_ball,
     [P.test_p1_lion_buffers_closed_form]),
    ("normalised by the largest entry", "frobenius_normalize", normalize_by_max,
     [P.test_p2_frobenius_unit_norm_and_zero]),
    ("sign of b flipped", "ns_direct_oriented", ns_sign_of_b_flipped,
     [lambda: P.test_p3_ns_scalar_map_on_singular_values(6, 10, COEFS[0])]),
    ("quintic term dropped", "ns_direct_oriented", ns_quintic_term_dropped,
     [lambda: P.test_p3_ns_scalar_map_on_singular_values(6, 10, COEFS[1])]),
    ("one iteration short", "ns_direct_oriented", ns_one_iteration_short,
     [lambda: P.test_p3_ns_scalar_map_on_singular_values(6, 10, COEFS[0])]),
    ("Gram update one-sided", "gram_ns_fresh_oriented", gram_one_sided_update,
     [lambda: P.test_p7_gram_equals_direct_and_q_properties(8, 20, COEFS[0])]),
    ("residual divided by r", "orth_residual", residual_over_r,
     [P.test_p8_residual_brute_force_and_special_values]),
    ("strict acceptance", "accept_cached", accept_strict,
     [P.test_p8_acceptance_is_inclusive]),
    ("zero counted negative", "sign_negative", sign_nonpositive,
     [P.test_p10_sign_special_values]),
    ("bits packed MSB first", "pack_bits", pack_msb_first,
     [lambda: P.test_p11_pack_brute_force(65)]),
    ("vote ties to +1", "vote_from_bits", vote_ties_positive,
     [lambda: P.test_p12_vote_brute_force_and_symmetries(4)]),
    ("update with the wrong sign", "update_vote", update_vote_wrong_sign,
     [P.test_p13_update_matches_torch_float32_and_bf16]),
    ("bf16 weights truncated", "update_vote", update_vote_bf16_truncated,
     [P.test_p13_update_matches_torch_float32_and_bf16, P.test_p13_hand_derived_bf16_values]),
    ("int8 sign of zero is zero", "sign_int8", sign_int8_zero_is_zero,
     [P.test_p16_sign_int8_special_values_and_payload]),
    ("int8 vote ties to +1", "vote_from_int8", vote_int8_ties_positive,
     [P.test_p16_int8_vote_ties_for_even_workers]),
    ("Muon phase shifted", "lion_muon_is_muon_step", muon_phase_shifted,
     [P.test_p14_schedule_phase]),
    ("Lion sign of the momentum alone", "lion_sign_negative", lion_sign_of_momentum_only,
     [P.test_lion_sign_is_the_exact_sign_of_the_interpolation]),
    ("polar update rounded once", "update_polar", update_polar_one_rounding,
     [P.test_update_polar_matches_torch_float32_and_bf16]),
    ("power method never normalised", "spectral_norm_power", power_without_normalising,
     [lambda: P.test_p18_power_method_converges_to_svd(30, 70), P.test_p18_power_method_closed_forms]),
    ("Frobenius norm for the spectral norm", "spectral_norm_power", power_frobenius,
     [lambda: P.test_p18_power_method_converges_to_svd(30, 70), P.test_p18_power_method_closed_forms]),
    ("tall matrices not transposed", "orient", orient_never_transposes,
     [P.test_p3_tall_orientation_matches_transpose_map, P.test_p7_gram_tall_orientation]),
    ("vote not normalised before its polar step", "vote_polar_direction", vote_polar_unnormalised,
     [lambda: P.test_p17_vote_polar_on_hadamard_votes_closed_form(COEFS[0], 8, 1, False),
      P.test_p17_vote_polar_rank_one_and_zero_votes]),
    ("bits unpacked MSB first", "unpack_bits", unpack_reversed,
     [lambda: P.test_p11_pack_brute_force(65), lambda: P.test_p12_vote_brute_force_and_symmetries(3)]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_planted_mistake_fails_a_pin(monkeypatch, case):
    _, name, mutant, pins = case
    assert hasattr(O, name)
    monkeypatch.setattr(O, name, mutant)
    failed = []
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin)
    assert failed, f"no pin caught the planted mistake in {name}"


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_pins_pass_on_the_oracle_itself(case):
    """The same pins pass with the oracle unchanged (so a failure above is
    the planted mistake's)."""
    for pin in case[3]:
        pin()
