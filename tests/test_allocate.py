"""TriAxialKV bit allocation in the library (oscar_allocate_bits, a host call) against the oracle's
greedy and brute force, and against an exact knapsack dynamic programme at 22 classes (an
independent method: the least distortion is the total at 2 bits minus the largest gain sum whose
extra bits fit the budget)."""
import ctypes

import numpy as np
import pytest

import bit_rotated_kv_amd as brk
import oracle
import problem as P
import synth
from bit_rotated_kv_amd import _lib


def _instance(r, k, int_counts=False, ties=False):
    d4 = r.uniform(0, 1, k)
    gain = r.uniform(-0.5, 5, k) if not ties else np.repeat(r.uniform(0.5, 5, (k + 1) // 2), 2)[:k]
    d2 = d4 + gain
    n = r.integers(0, 200, k) if not ties else np.repeat(r.integers(1, 50, (k + 1) // 2), 2)[:k]
    if int_counts:
        n = r.integers(1, 120, k)
    return d2, d4, n.astype(np.int64)


def cost(bits, d2, d4):
    return float(np.where(np.asarray(bits) == 4, d4, d2).sum())


def test_greedy_matches_the_oracle():
    r = np.random.default_rng(50)
    for trial in range(400):
        k = int(r.integers(1, 57))
        d2, d4, n = _instance(r, k, ties=trial % 3 == 0)
        budget = float(r.uniform(2.0, 4.2))
        got, c = brk.allocate_bits(d2, d4, n, budget, "greedy")
        ref = oracle.greedy_bit_allocation(d2, d4, n, budget)
        assert np.array_equal(got, ref), (trial, k)
        assert np.isclose(c, cost(ref, d2, d4))


def test_exhaustive_matches_the_oracle_brute_force():
    r = np.random.default_rng(51)
    for trial in range(60):
        k = int(r.integers(1, 11))
        d2, d4, n = _instance(r, k)
        budget = float(r.uniform(2.0, 3.8))
        got, c = brk.allocate_bits(d2, d4, n, budget, "exhaustive")
        ref = oracle.exhaustive_bit_allocation(d2, d4, n, budget)
        assert (got.astype(np.int64) * n).sum() <= budget * n.sum() + 1e-9
        assert np.isclose(cost(got, d2, d4), cost(ref, d2, d4), rtol=1e-12, atol=1e-12)
        assert np.isclose(c, cost(got, d2, d4))


def _knapsack_optimum(d2, d4, n, budget):
    """Least total distortion by dynamic programming over integer extra-bit weights."""
    cap = int(np.floor(budget * n.sum() + 1e-9)) - 2 * int(n.sum())
    best = np.full(cap + 1, -np.inf)
    best[0] = 0.0
    for k in range(len(n)):
        g, wk = d2[k] - d4[k], 2 * int(n[k])
        if wk > cap:
            continue
        upd = best[: cap + 1 - wk] + g
        best[wk:] = np.maximum(best[wk:], upd)
    return float(d2.sum() - best.max())


def test_exhaustive_at_22_classes_is_the_knapsack_optimum():
    r = np.random.default_rng(52)
    for trial in range(6):
        d2, d4, n = _instance(r, 22, int_counts=True)
        budget = float(r.uniform(2.2, 3.2))
        got, c = brk.allocate_bits(d2, d4, n, budget, "exhaustive")
        assert (got.astype(np.int64) * n).sum() <= budget * n.sum() + 1e-9
        assert np.isclose(c, _knapsack_optimum(d2, d4, n, budget), rtol=1e-12, atol=1e-12)
        g, gc = brk.allocate_bits(d2, d4, n, budget, "greedy")
        assert c <= gc + 1e-12


def test_workload_allocation_matches_the_oracle():
    """The mixed workload's class widths: the library's greedy equals the oracle's, spending close to
    the 2.6-bit budget (about 30% of the tokens at 4 bits); the exhaustive optimum is no worse."""
    w = synth.workload(5)
    d2, d4 = synth.tag_sensitivity(w)
    n = synth.tag_nominal_counts(w)
    got, c = brk.allocate_bits(d2, d4, n, w.bit_budget)
    assert np.array_equal(got, P.class_bits(w))
    share = (n * (got == 4)).sum() / n.sum()
    assert 0.25 < share <= 0.30
    e, ec = brk.allocate_bits(d2, d4, n, w.bit_budget, "exhaustive")
    assert ec <= c + 1e-15


def test_allocation_argument_checks():
    L = _lib.lib()
    one = np.ones(3)
    cnt = np.ones(3, np.int64)
    out = np.zeros(3, np.uint8)
    p = lambda a: a.ctypes.data
    assert L.oscar_allocate_bits(3, p(one), p(one), p(cnt), 1.9, 0, p(out), None) == -1     # budget below 2
    assert L.oscar_allocate_bits(3, p(one), p(one), p(cnt), float("nan"), 0, p(out), None) == -1
    assert L.oscar_allocate_bits(3, p(one), p(one), p(cnt), 3.0, 2, p(out), None) == -1     # method
    assert L.oscar_allocate_bits(3, None, p(one), p(cnt), 3.0, 0, p(out), None) == -1
    neg = np.array([1, -1, 1], np.int64)
    assert L.oscar_allocate_bits(3, p(one), p(one), p(neg), 3.0, 0, p(out), None) == -1
    big = np.ones(25)
    bc = np.ones(25, np.int64)
    bo = np.zeros(25, np.uint8)
    assert L.oscar_allocate_bits(25, p(big), p(big), p(bc), 3.0, 1, p(bo), None) == -2     # exhaustive > 24
    assert L.oscar_allocate_bits(0, None, None, None, 3.0, 1, None, None) == 0
    assert L.oscar_route_tokens(1, 10, 1, 1, 65, 1, 1, None) == -1                         # > 64 classes
    assert L.oscar_route_tokens(0, 10, None, None, 3, None, None, None) == 0
    bad = np.array([2, 3], np.uint8)
    assert L.oscar_route_tokens(1, 10, 1, 1, 2, p(bad), 1, None) == -1                      # width 3
