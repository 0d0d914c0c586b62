"""Pins of the TriAxialKV bit allocation in the oracle (no GPU)."""
import numpy as np

import oracle


def test_budget_extremes():
    d2, d4, n = [5.0, 3.0, 1.0], [1.0, 1.0, 0.5], [10, 20, 30]
    assert list(oracle.greedy_bit_allocation(d2, d4, n, 2.0)) == [2, 2, 2]
    assert list(oracle.greedy_bit_allocation(d2, d4, n, 4.0)) == [4, 4, 4]
    assert list(oracle.exhaustive_bit_allocation(d2, d4, n, 4.0)) == [4, 4, 4]


def test_greedy_order_by_gain_per_bit():
    # gains per 2N bits: class0 4/20=0.2, class1 2/40=0.05, class2 0.5/60
    d2, d4, n = [5.0, 3.0, 1.0], [1.0, 1.0, 0.5], [10, 20, 30]
    budget = (2 * 60 + 2 * 10) / 60.0          # room for class 0 only
    assert list(oracle.greedy_bit_allocation(d2, d4, n, budget)) == [4, 2, 2]


def test_greedy_equals_exhaustive_with_equal_counts():
    r = np.random.default_rng(40)
    for trial in range(20):
        k = 8
        d4 = r.uniform(0, 1, k)
        d2 = d4 + r.uniform(0, 5, k)
        n = np.full(k, 100)
        budget = 2 + 2 * r.integers(0, k + 1) / k
        g = oracle.greedy_bit_allocation(d2, d4, n, budget)
        e = oracle.exhaustive_bit_allocation(d2, d4, n, budget)
        cost = lambda b: np.where(b == 2, d2, d4).sum()
        assert np.isclose(cost(g), cost(e))
        assert (g * n).sum() <= budget * n.sum() + 1e-9


def test_exhaustive_is_feasible_and_no_worse():
    r = np.random.default_rng(41)
    for trial in range(20):
        k = 7
        d4 = r.uniform(0, 1, k)
        d2 = d4 + r.uniform(0, 5, k)
        n = r.integers(1, 200, k)
        budget = r.uniform(2.0, 3.5)
        g = oracle.greedy_bit_allocation(d2, d4, n, budget)
        e = oracle.exhaustive_bit_allocation(d2, d4, n, budget)
        cost = lambda b: np.where(b == 2, d2, d4).sum()
        assert (e * n).sum() <= budget * n.sum() + 1e-9
        assert cost(e) <= cost(g) + 1e-12
