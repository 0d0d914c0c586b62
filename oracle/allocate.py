"""INT2/INT4 bit allocation over tag classes (oracle).

Follows the TriAxialKV reading note (section 3, "greedy or exhaustive"): minimise
sum_k D_k(b_k) subject to sum_k N_k b_k <= B sum_k N_k with b_k in {2, 4}. Raising class k
from 2 to 4 bits costs 2 N_k bits and gains D_k(2) - D_k(4); the greedy visits classes by
descending rho_k = (D_k(2) - D_k(4)) / (2 N_k) and raises them until the budget is spent.
For small class counts the note says exhaustive search over 2^K configurations is
affordable.

Readings: only classes with a positive gain are raised; the greedy stops at the first
class whose raise would exceed the budget (the plain reading of "until the budget is
used up"); ties in rho keep the lower class index first.
"""
from __future__ import annotations

import itertools

import numpy as np


def greedy_bit_allocation(d2, d4, counts, budget_bits):
    """Bits per class (array of 2/4) from the greedy rule."""
    d2 = np.asarray(d2, np.float64)
    d4 = np.asarray(d4, np.float64)
    n = np.asarray(counts, np.float64)
    bits = np.full(len(n), 2, np.int64)
    allowed = budget_bits * n.sum()
    used = 2.0 * n.sum()
    rho = (d2 - d4) / (2.0 * np.maximum(n, 1e-300))
    order = sorted(range(len(n)), key=lambda k: (-rho[k], k))
    for k in order:
        if d2[k] - d4[k] <= 0 or n[k] == 0:
            continue
        if used + 2.0 * n[k] > allowed + 1e-9:
            break
        bits[k] = 4
        used += 2.0 * n[k]
    return bits


def exhaustive_bit_allocation(d2, d4, counts, budget_bits):
    """Bits per class minimising the total distortion among all feasible 2/4 choices
    (brute force; ties keep the configuration enumerated first)."""
    d2 = np.asarray(d2, np.float64)
    d4 = np.asarray(d4, np.float64)
    n = np.asarray(counts, np.float64)
    allowed = budget_bits * n.sum()
    best, best_cost = None, np.inf
    for choice in itertools.product((2, 4), repeat=len(n)):
        c = np.array(choice)
        if (c * n).sum() > allowed + 1e-9:
            continue
        cost = np.where(c == 2, d2, d4).sum()
        if cost < best_cost - 1e-15:
            best, best_cost = c, cost
    return best
