"""Pins of the oracle's adaptive (top-p) token budget against what fixes it
independently of the oracle's code: hand-computed shares, a geometric closed
form, a brute-force search over every subset, the softmax's +inf limit, and
the fixed-budget selection it must reduce to.

Reading under test (RaBitQCache abstract, second page: top-p retrieval in
place of a fixed top-k): the selection is the smallest set of candidates whose
softmax shares (over all candidates t < L) reach top_p, cut at the budget;
among sets of that size the top-ranked one (score descending, lower index
first) is taken.
"""

import itertools
import math

import numpy as np
import pytest

from oracle import decode as O


def _sel(scores, budget, p, seq_len=None):
    scores = np.asarray(scores, dtype=np.float64)
    idx, n = O.select_tokens_top_p(scores, len(scores) if seq_len is None else seq_len, budget, p)
    return [int(x) for x in idx[:n]], n


def test_hand_computed_shares():
    # shares 1, 3, 2, 4 (out of 10): ranked 3 (0.4), 1 (0.3), 2 (0.2), 0 (0.1)
    s = np.log([1.0, 3.0, 2.0, 4.0])
    assert _sel(s, 4, 0.35) == ([3], 1)
    assert _sel(s, 4, 0.65) == ([1, 3], 2)
    assert _sel(s, 4, 0.75) == ([1, 2, 3], 3)
    assert _sel(s, 4, 0.95) == ([0, 1, 2, 3], 4)
    assert _sel(s, 2, 0.95) == ([1, 3], 2)  # the budget caps it
    # a constant added to every logit changes no share
    assert _sel(s + 1000.0, 4, 0.65) == ([1, 3], 2)
    assert _sel(s - 1000.0, 4, 0.75) == ([1, 2, 3], 3)


def test_geometric_closed_form():
    # weights 2^-k at shuffled positions: the top k hold (1 - 2^-k) / (1 - 2^-n)
    n = 40
    rng = np.random.default_rng(3)
    pos = rng.permutation(n)
    s = np.empty(n)
    s[pos] = -np.arange(n) * math.log(2.0)
    for p in (0.3, 0.6, 0.9, 0.99):
        k = next(k for k in range(1, n + 1) if 1 - 2.0 ** -k >= p * (1 - 2.0 ** -n))
        got, cnt = _sel(s, n, p)
        assert cnt == k, (p, cnt, k)
        assert got == sorted(int(x) for x in pos[:k])


def test_equal_scores_take_the_lowest_indices():
    # n equal logits: ceil(p n) of them, the lowest indices
    for n, p in ((10, 0.25), (10, 0.3), (7, 0.5), (128, 0.9)):
        k = math.ceil(p * n - 1e-12)
        assert _sel(np.full(n, 0.7), n, p) == (list(range(k)), k)


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_smallest_subset(seed):
    # every subset of a tiny row: the smallest size whose best subset reaches p,
    # then the best-ranked subset of that size
    rng = np.random.default_rng(seed)
    n = 7
    s = rng.standard_normal(n) * 2.0
    w = np.exp(s - s.max())
    z = w.sum()
    for p in (0.2, 0.5, 0.8, 0.97):
        for budget in (2, 4, 7):
            size = None
            for k in range(1, n + 1):
                if max(w[list(c)].sum() for c in itertools.combinations(range(n), k)) >= p * z:
                    size = k
                    break
            size = min(size, budget, n)
            best = max(itertools.combinations(range(n), size),
                       key=lambda c: (sorted(s[list(c)], reverse=True), [-i for i in c]))
            assert _sel(s, budget, p) == (sorted(best), size), (seed, p, budget)


def test_positive_infinity_takes_the_whole_mass():
    s = [0.0, np.inf, 5.0, np.inf]
    assert _sel(s, 4, 0.4) == ([1], 1)
    assert _sel(s, 4, 0.6) == ([1, 3], 2)
    assert _sel(s, 4, 1.0) == ([1, 3], 2)


def test_nan_and_minus_infinity_weigh_nothing():
    s = [np.nan, 0.0, -np.inf, np.log(3.0), np.nan]
    # shares: token 3: 0.75, token 1: 0.25
    assert _sel(s, 5, 0.7) == ([3], 1)
    assert _sel(s, 5, 0.9) == ([1, 3], 2)
    assert _sel(s, 5, 1.0) == ([1, 3], 2)


def test_no_weight_or_top_p_zero_keeps_the_fixed_budget():
    rng = np.random.default_rng(5)
    s = rng.standard_normal(300)
    for budget in (1, 17, 300, 400):
        fixed = O.select_tokens_unit(s, 300, budget)
        got = O.select_tokens_top_p(s, 300, budget, 0.0)
        assert np.array_equal(got[0], fixed[0]) and got[1] == fixed[1]
    nan_row = np.full(50, np.nan)
    got = O.select_tokens_top_p(nan_row, 50, 8, 0.5)
    fixed = O.select_tokens_unit(nan_row, 50, 8)
    assert np.array_equal(got[0], fixed[0]) and got[1] == fixed[1] == 8
    minus = np.full(20, -np.inf)
    assert O.select_tokens_top_p(minus, 20, 6, 0.5)[1] == 6


def test_only_the_first_seq_len_candidates_count():
    s = np.log([1.0, 1.0, 8.0, 100.0])
    # with L = 3 the 100 is no candidate: shares 0.1, 0.1, 0.8
    assert _sel(s, 4, 0.75, seq_len=3) == ([2], 1)
    assert _sel(s, 4, 0.85, seq_len=3) == ([0, 2], 2)
    assert _sel(s, 4, 0.5, seq_len=0) == ([], 0)
