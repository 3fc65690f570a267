"""Pins of the oracle's selection policies (S1): budget, sparsity ratio, threshold.

Source: "SeerAttention: Learning Intrinsic Sparse Attention in Your LLMs",
abstract v2 (the gate adapts to varying context lengths and sparsity ratios);
"SeerAttention-R", abstract (a token budget).  Readings (R23): the ratio
policy keeps ceil(nc * num / den) blocks; the threshold policy keeps the
blocks whose softmax probability over the (b, KV head)'s block scores is at
least tau; both are capped by the row width k_max and use D4's top-k rule
(ties toward the lower id, ids ascending).  Pins: counts in closed form, the
definition evaluated independently with numpy, brute force over subsets, and
the budget policy equal to the plain selection.
"""
import itertools
import math

import numpy as np
import pytest

import oracle


def rng_scores(n, seed, ties=False):
    r = np.random.default_rng(seed)
    if ties:
        return r.integers(-3, 4, size=n).astype(np.float64)
    return r.standard_normal(n)


@pytest.mark.parametrize("nc,num,den,expect", [(512, 1, 10, 52), (7, 1, 3, 3), (0, 1, 10, 0), (10, 1, 10, 1),
                                                (11, 1, 10, 2), (100, 0, 5, 0), (5, 7, 3, 5), (300, 1, 1, 300)])
def test_ratio_counts_closed_form(nc, num, den, expect):
    S = rng_scores(nc, nc)
    idx = oracle.select_policy(S, oracle.POLICY_RATIO, 10_000, num, den)
    assert len(idx) == expect


@pytest.mark.parametrize("nc,k_max", [(40, 8), (40, 100), (1, 1), (0, 5)])
def test_budget_policy_equals_plain_selection(nc, k_max):
    S = rng_scores(nc, 3 * nc + k_max, ties=True)
    a = oracle.select_policy(S, oracle.POLICY_BUDGET, k_max)
    b = oracle.select_blocks(S, k_max)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("nc,tau", [(64, 0.02), (64, 0.005), (200, 0.01), (10, 0.5), (10, 2.0), (10, 0.0),
                                    (10, -1.0)])
def test_threshold_keeps_the_blocks_above_tau(nc, tau):
    S = rng_scores(nc, nc + 17) * 2.0
    idx = oracle.select_policy(S, oracle.POLICY_THRESHOLD, 10_000, tau=tau)
    p = np.exp(S - S.max())
    p /= p.sum()
    expect = np.flatnonzero(p >= tau)          # already ascending
    assert np.array_equal(idx, expect)


def test_threshold_capped_by_row_width_takes_the_best():
    S = rng_scores(100, 5)
    idx = oracle.select_policy(S, oracle.POLICY_THRESHOLD, 6, tau=0.0)  # every block passes, 6 fit
    assert np.array_equal(idx, np.sort(np.argsort(-S, kind="stable")[:6]))


def test_threshold_equal_scores_all_or_nothing():
    S = np.full(20, 1.5)
    assert len(oracle.select_policy(S, oracle.POLICY_THRESHOLD, 100, tau=0.05)) == 20   # p = 1/20
    assert len(oracle.select_policy(S, oracle.POLICY_THRESHOLD, 100, tau=0.0500001)) == 0
    capped = oracle.select_policy(S, oracle.POLICY_THRESHOLD, 7, tau=0.01)
    assert np.array_equal(capped, np.arange(7))   # ties go to the lower ids


@pytest.mark.parametrize("seed", range(6))
def test_ratio_set_is_a_best_subset_brute_force(seed):
    S = rng_scores(9, seed, ties=seed % 2 == 0)
    idx = oracle.select_policy(S, oracle.POLICY_RATIO, 100, 1, 3)
    k = 3
    best = max(itertools.combinations(range(9), k), key=lambda c: (sum(S[list(c)]), [-x for x in c]))
    assert sorted(best) == list(idx)


def test_bad_arguments_rejected():
    with pytest.raises((RuntimeError, ValueError)):
        oracle.select_policy([1.0, 2.0], 7, 2)
    with pytest.raises((RuntimeError, ValueError)):
        oracle.select_policy([1.0, 2.0], oracle.POLICY_RATIO, 2, 1, 0)
