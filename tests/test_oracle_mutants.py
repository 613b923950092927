"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in the oracle (a dropped term, a wrong sign,
weight, comparison or operand order) by replacing one of its functions for
the duration of the test, then runs the pins that should notice it; at
least one must fail.  The oracle module itself is never edited: the
replacement goes through pytest's monkeypatch, so every later test sees the
real oracle again.
"""

import math

import numpy as np
import pytest

from oracle import solattn_ref as ref
from tests import test_oracle_pins as pins

REAL = {name: getattr(ref, name) for name in (
    "pool", "key_moments", "thresholds", "select", "proxy_scores", "block_sizes",
    "first_order_terms", "kv_moments", "order_row", "dense", "row_stats")}


def vhat_as_mean(q, k, v, block):
    qbar, kbar, vhat = REAL["pool"](q, k, v, block)
    n = REAL["block_sizes"](q.shape[0], block).astype(np.float64)
    return qbar, kbar, vhat / n[:, None]


def sample_covariance(kbar):
    m, cov = REAL["key_moments"](kbar)
    N = kbar.shape[0]
    return m, cov * N / max(N - 1, 1)


def tau_minus(mu, sigma, beta):
    return REAL["thresholds"](mu, sigma, -beta)


def strict_select(shat, tau):
    return np.asarray(shat) > np.asarray(tau)[:, None]


def unscaled_proxy(qbar, kbar, scale):
    return REAL["proxy_scores"](qbar, kbar, 1.0)


def unit_block_weights(L, block):
    return np.ones_like(REAL["block_sizes"](L, block))


def doubled_block_weights(L, block):
    return 2 * REAL["block_sizes"](L, block)


def first_order_sign(qi, kj, vj, centre, ref_max, scale):
    num, den = REAL["first_order_terms"](qi, kj, vj, centre, ref_max, scale)
    return -num, den


def first_order_twice(qi, kj, vj, centre, ref_max, scale):
    num, den = REAL["first_order_terms"](qi, kj, vj, centre, ref_max, scale)
    return 2.0 * num, den


def kv_moments_transposed(k, v, block):
    return np.transpose(REAL["kv_moments"](k, v, block), (0, 2, 1))


def ties_by_decreasing_index(shat_row):
    s = np.asarray(shat_row, np.float64)
    return np.lexsort((-np.arange(s.size), -s))


def dense_without_scale(q, k, v, scale):
    return REAL["dense"](q, k, v, 1.0)


def row_stats_variance(qbar, m, cov, scale):
    mu, sigma = REAL["row_stats"](qbar, m, cov, scale)
    return mu, sigma * sigma


def run_pins(calls):
    failed = []
    for call in calls:
        try:
            call()
        except AssertionError:
            failed.append(call)
    return failed


P = pins
MUTANTS = {
    # name: (function replaced, replacement, pins expected to notice)
    "vhat_is_a_mean": ("pool", vhat_as_mean, [
        lambda: P.test_pool_matches_numpy_segment_reductions(1000),
        lambda: P.test_block_constant_keys_make_the_approximation_exact(1.0),
        P.test_hand_worked_example]),
    "sample_covariance": ("key_moments", sample_covariance, [
        lambda: P.test_row_stats_equal_bruteforce_proxy_rows("iid_ragged"),
        P.test_hand_worked_example]),
    "tau_below_mu": ("thresholds", tau_minus, [
        lambda: P.test_mean_density_tracks_gaussian_tail(1.0),
        P.test_hand_worked_example]),
    "strict_comparison": ("select", strict_select, [
        P.test_two_blocks_put_tau_on_the_larger_score,
        P.test_hand_worked_example]),
    "proxy_without_scale": ("proxy_scores", unscaled_proxy, [
        lambda: P.test_row_stats_equal_bruteforce_proxy_rows("iid_ragged"),
        P.test_hand_worked_example]),
    "no_block_weight": ("block_sizes", unit_block_weights, [
        lambda: P.test_block_constant_keys_make_the_approximation_exact(1.0),
        P.test_beta_plus_inf_is_attention_over_pooled_keys]),
    "doubled_block_weight": ("block_sizes", doubled_block_weights, [
        P.test_approx_denominator_is_below_the_exact_one]),
    "first_order_sign": ("first_order_terms", first_order_sign, [
        P.test_first_order_error_is_second_order_in_the_key_spread,
        P.test_hand_worked_example]),
    "first_order_doubled": ("first_order_terms", first_order_twice, [
        P.test_first_order_error_is_second_order_in_the_key_spread,
        P.test_kv_moments_give_the_first_order_numerator]),
    "kv_moments_transposed": ("kv_moments", kv_moments_transposed, [
        P.test_kv_moments_is_n_times_numpy_cross_covariance,
        P.test_kv_moments_give_the_first_order_numerator]),
    "topk_ties_reversed": ("order_row", ties_by_decreasing_index, [
        P.test_topk_breaks_ties_by_block_index]),
    "dense_without_scale": ("dense", dense_without_scale, [
        lambda: P.test_beta_minus_inf_is_dense_attention(1000)]),
    "sigma_is_a_variance": ("row_stats", row_stats_variance, [
        lambda: P.test_row_stats_equal_bruteforce_proxy_rows("pos"),
        P.test_hand_worked_example]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    target, replacement, calls = MUTANTS[name]
    # the real pins pass
    assert not run_pins(calls), "a pin fails on the real oracle"
    monkeypatch.setattr(ref, target, replacement)
    assert run_pins(calls), f"no pin noticed the planted mistake {name!r}"
