"""Pins of the oracle's top-k page selection.

Brute force: on small rows with many exact ties, the selection equals the
reserved pages plus the first k-|R| pages of a full Python sort by
(score desc, index asc).  Special cases: k >= N keeps every page, k = 1 keeps
only the tail, equal scores keep the tail plus the lowest indices, and the
budget formula with a fraction and a floor.
"""
import math

import numpy as np

import oracle


def _brute(scores, k_pages, frac, bos, eos):
    N = len(scores)
    k = min(N, max(k_pages, math.floor(frac * N)))
    lo, hi = min(bos, N), max(N - eos, 0)
    hi = max(hi, lo)
    reserved = [p for p in range(N) if p < lo or p >= hi]
    rest = sorted(range(lo, hi), key=lambda p: (-scores[p], p))
    take = rest[:max(0, k - len(reserved))]
    return sorted(reserved + take)


def test_selection_brute_force_with_ties():
    rng = np.random.default_rng(0)
    for trial in range(400):
        N = int(rng.integers(1, 60))
        scores = rng.integers(-4, 5, size=N).astype(np.float64)   # many ties
        if trial % 3 == 0:
            scores = rng.standard_normal(N)
        k = int(rng.integers(1, N + 3))
        frac = float(rng.choice([0.0, 0.1, 0.37]))
        bos = int(rng.integers(0, 4))
        eos = int(rng.integers(0, 4))
        got = oracle.select(scores, k, frac, bos, eos).tolist()
        assert got == _brute(list(scores), k, frac, bos, eos), (N, k, frac, bos, eos)


def test_all_pages_when_budget_covers_row():
    s = np.random.default_rng(1).standard_normal(17)
    assert oracle.select(s, 17).tolist() == list(range(17))
    assert oracle.select(s, 50).tolist() == list(range(17))


def test_budget_one_is_tail_only():
    s = np.arange(10, dtype=np.float64)[::-1].copy()   # page 0 scores highest
    assert oracle.select(s, 1).tolist() == [9]


def test_equal_scores_take_lowest_indices_plus_tail():
    s = np.zeros(12)
    assert oracle.select(s, 4).tolist() == [0, 1, 2, 11]


def test_tail_counts_in_budget_and_top_scores_win():
    s = np.array([0.1, 5.0, 0.2, 4.0, 0.3, -9.0])
    # budget 3 = tail (page 5) + the two best of pages 0..4
    assert oracle.select(s, 3).tolist() == [1, 3, 5]


def test_budget_formula():
    assert oracle.budget(100, 4, 0.1) == 10
    assert oracle.budget(39, 4, 0.1) == 4          # floor(3.9) = 3 < 4
    assert oracle.budget(3, 4, 0.1) == 3           # capped at N
    assert oracle.budget(2050, 4, 0.1) == 205
    assert oracle.budget(8192, 256) == 256


def test_reserved_exceeding_budget_are_all_kept():
    s = np.random.default_rng(2).standard_normal(10)
    assert oracle.select(s, 2, 0.0, 3, 2).tolist() == [0, 1, 2, 8, 9]
