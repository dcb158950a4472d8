"""Pins of the oracle's choice of k ("How Speculative Decoding Speeds Up
Inference", section "Tokens per pass and time per token", Eq. (1) and (2)).

What fixes the expected values:
  * Eq. (1) against the geometric series sum_j alpha^j (slot j is reached
    with probability alpha^j under the page's independence) and against the
    page's statements (tests/golden/eq1_page_statements.json);
  * the marginal condition stated on the SparseSpec-L page: a longer horizon
    stops paying when the marginal acceptance probability falls below the
    relative drafting cost. From Eq. (2), t(k+1) < t(k) exactly when
    alpha^(k+1) > t_draft * E_k / (t_pass + k t_draft); with a constant pass
    time the chosen k is the first k where that fails;
  * limits: no speculation at alpha = 0, the longest horizon when drafting is
    free, and the blog's qualitative claim that long drafts pay only when the
    draft is usually right;
  * the acceptance-rate estimate on rounds drawn with a planted alpha, and its
    prior and decay limits.
"""
import json
import os

import numpy as np
import pytest

from nested_quantized_weights_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("alpha", [0.0, 0.1, 0.5, 0.66, 0.9, 0.95, 0.999, 1.0])
@pytest.mark.parametrize("k", [0, 1, 4, 8, 16])
def test_eq1_is_the_geometric_series(oracle, alpha, k):
    series = sum(alpha ** j for j in range(k + 1))
    assert abs(oracle.expected_tokens(alpha, k) - series) <= 1e-12 * max(1.0, series)


def test_eq1_page_statements(oracle):
    ex = json.load(open(os.path.join(GOLDEN, "eq1_page_statements.json")))
    s05, s09 = ex["statements"]
    e = oracle.expected_tokens
    assert e(s05["alpha"], s05["k_long"]) - e(s05["alpha"], s05["k_short"]) < 0.1  # "add little"
    assert abs(e(s09["alpha"], s09["k_long"]) - e(s09["alpha"], s09["k_short"]) - 2.0) < 0.1  # "about 2"


def test_eq2_time_per_token(oracle):
    # one pass of 20 s and drafts of 30 ms (the blog's laptop numbers), alpha = 0.5, k = 8
    t = oracle.token_time(0.5, 8, 0.03, 20.0)
    assert abs(t - (20.0 + 8 * 0.03) / oracle.expected_tokens(0.5, 8)) < 1e-12
    assert oracle.token_time(0.0, 0, 1.0, 7.0) == 7.0  # no speculation: one token per pass


@pytest.mark.parametrize("ratio", [0.002, 0.05, 0.2, 0.6])
def test_choice_follows_the_marginal_condition(oracle, ratio):
    kmax = 32
    t_pass = np.ones(kmax + 1)
    for alpha in np.linspace(0.0, 0.99, 34):
        k = oracle.choose_k(alpha, ratio, t_pass)
        # the first k at which one more draft stops paying
        first = kmax
        for j in range(kmax):
            if not alpha ** (j + 1) > ratio * oracle.expected_tokens(alpha, j) / (1.0 + j * ratio):
                first = j
                break
        assert k == first, (alpha, ratio, k, first)


def test_choice_limits_and_monotonicity(oracle):
    kmax = 16
    t_pass = np.ones(kmax + 1)
    assert oracle.choose_k(0.0, 0.01, t_pass) == 0
    assert oracle.choose_k(0.5, 0.0, t_pass) == kmax  # free drafting never hurts
    assert oracle.choose_k(1.0, 0.5, t_pass) == kmax  # always accepted, drafting cheaper than a pass
    ks = [oracle.choose_k(a, 0.05, t_pass) for a in np.linspace(0, 0.99, 50)]
    assert all(a <= b for a, b in zip(ks, ks[1:]))
    # long drafts are worth it only at a high acceptance rate (blog, "Tokens per
    # pass and time per token")
    assert oracle.choose_k(0.5, 0.05, t_pass) <= 4 < 8 <= oracle.choose_k(0.9, 0.05, t_pass)
    # a pass that grows with k moves the choice down
    growing = 1.0 + 0.05 * np.arange(kmax + 1)
    assert oracle.choose_k(0.9, 0.05, growing) < oracle.choose_k(0.9, 0.05, t_pass)


@pytest.mark.parametrize("alpha,k", [(0.58, 8), (0.66, 4), (0.95, 8)])
def test_alpha_estimate_on_planted_rounds(oracle, alpha, k):
    g = synth.rng(600, int(alpha * 100), k)
    R = 20000
    # accepted slots of a round: geometric, truncated at k
    acc = np.minimum(g.geometric(1.0 - alpha, size=R) - 1, k)
    est = oracle.alpha_estimate(acc, k, prior_accepted=0.0, prior_rejected=0.0)
    judged = acc.sum() + (acc < k).sum()
    sd = np.sqrt(alpha * (1 - alpha) / judged)
    assert abs(est - alpha) < 4 * sd


def test_alpha_estimate_prior_and_decay(oracle):
    assert oracle.alpha_estimate(np.zeros(0, np.int64), 4, prior_accepted=3.0, prior_rejected=1.0) == 0.75
    assert oracle.alpha_estimate([4, 4, 4], 4, prior_accepted=0.0, prior_rejected=0.0) == 1.0
    # decay 0: only the last round counts (2 accepted, then a rejection)
    assert oracle.alpha_estimate([4, 0, 2], 4, decay=0.0) == pytest.approx(2 / 3)
