"""The library's host functions for choosing k (nest_expected_tokens,
nest_token_time, nest_choose_k, nest_alpha_*) against the oracle's, on the
CPU (these functions never touch the GPU). Expected tokens agree to 1e-12
relative (the library sums the series, the oracle evaluates the closed
form); the chosen k and the acceptance estimates agree exactly.
"""
import os

import numpy as np
import pytest

from nested_quantized_weights_amd import synth

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "nested_quantized_weights_amd", "libnestspec.so")


@pytest.fixture(scope="module")
def ns():
    if not os.path.exists(LIB):
        pytest.skip("libnestspec.so not built (run __graft_entry__.build())")
    from nested_quantized_weights_amd import nestspec

    return nestspec


def test_expected_tokens_and_time(ns, oracle):
    for alpha in np.linspace(0.0, 1.0, 41):
        for k in range(0, 20):
            e, o = ns.expected_tokens(alpha, k), oracle.expected_tokens(alpha, k)
            assert abs(e - o) <= 1e-12 * o
            assert abs(ns.token_time(alpha, k, 0.03, 1.7) - oracle.token_time(alpha, k, 0.03, 1.7)) <= 1e-12
    assert np.isnan(ns.expected_tokens(1.5, 3)) and np.isnan(ns.expected_tokens(0.5, -1))


def test_choose_k_matches_oracle(ns, oracle):
    g = synth.rng(610)
    for _ in range(300):
        kmax = int(g.integers(0, 17))
        t_pass = np.sort(g.uniform(0.5, 2.0, kmax + 1))  # a pass grows with k
        t_draft = float(g.uniform(0.0, 0.5))
        alpha = float(g.uniform(0.0, 1.0))
        k, t = ns.choose_k(alpha, t_draft, t_pass)
        assert k == oracle.choose_k(alpha, t_draft, t_pass)
        assert abs(t - oracle.token_time(alpha, k, t_draft, t_pass[k])) <= 1e-12 * t


def test_choose_k_rejects_bad_arguments(ns):
    with pytest.raises(ns.NestError):
        ns.choose_k(1.2, 0.1, [1.0, 1.0])


def test_alpha_estimate_matches_oracle(ns, oracle):
    g = synth.rng(611)
    for decay in (1.0, 0.9, 0.0):
        k = 8
        acc = np.minimum(g.geometric(0.3, size=500) - 1, k)
        est = ns.AlphaEstimate(decay=decay, prior_accepted=2.0, prior_rejected=1.0)
        for a in acc:
            est.update(int(a), k)
        assert est.value == oracle.alpha_estimate(acc, k, decay=decay, prior_accepted=2.0, prior_rejected=1.0)
