"""FreeBalance's budgeted expert-swap planner (test infrastructure only, like
the rest of ``oracle/``).

Source: FreeBalance ("FreeBalance: Pre-Routing Online MoE Load Balancing via
Residual Workload Prediction"), section 3.3 "Budgeted Expert-Swap Planning",
eq. 6-8 and 10, and Algorithm 1.

* Workload: n_e = predicted pairs of expert e (column sums of the predicted
  count matrix, eq. 5); a rank's load is the sum over the experts it holds
  (no replicas: every pair of e runs where e lives).
* A swap of e_a (on rank a) with e_b (on rank b) changes only those two
  loads (eq. 6-7): L_a' = L_a - n_a + n_b, L_b' = L_b - n_b + n_a.
* Objective (eq. 8): Phi(L) = max_r L_r + gamma * sum_r (L_r - mean)^2; the
  benefit of a swap is Phi(L) - Phi(L'); non-positive benefits are dropped.
* Algorithm 1: while the most- and least-loaded ranks differ by more than
  tau and budget remains, take a beneficial swap between them; stop when
  none exists.

Readings (the page leaves these open):
* Candidates each step are the pairs (e_a on the most-loaded rank a, e_b on
  the least-loaded rank b) -- the frontier the page says the planner uses in
  practice; ranks tie to the lower index.
* Every swap moves two equal-sized experts over one intra-node link, so the
  cost model (eq. 9) gives every swap the same cost and the budget (eq. 10)
  becomes a number of swaps per rank; benefit-to-cost order is then benefit
  order.  Ties: lower e_a, then lower e_b (layer and ranks are fixed within
  a step).
* An expert moved once is not moved again ("neither expert has already been
  selected").
* gamma is a non-negative rational num/den, so every comparison is exact.
  Since the mean is unchanged by a swap, the variance term of the benefit is
  2*d*(L_a - L_b - d) with d = n_a - n_b (checked against eq. 8 directly in
  the tests).
"""
from __future__ import annotations

from fractions import Fraction
from typing import List, Sequence, Tuple

import numpy as np


def phi(load: Sequence[int], gamma: Fraction) -> Fraction:
    """Eq. 8, exactly."""
    G = len(load)
    mean = Fraction(sum(int(v) for v in load), G)
    return max(int(v) for v in load) + gamma * sum((int(v) - mean) ** 2 for v in load)


def swap_benefit(load: Sequence[int], a: int, b: int, n_a: int, n_b: int, gamma: Fraction) -> Fraction:
    """Phi(L) - Phi(L') for the swap of an expert with n_a pairs on rank a and
    one with n_b pairs on rank b, in closed form."""
    d = n_a - n_b
    new_a, new_b = load[a] - d, load[b] + d
    other = max((int(load[r]) for r in range(len(load)) if r not in (a, b)), default=None)
    m_new = max(new_a, new_b) if other is None else max(new_a, new_b, other)
    return (max(int(v) for v in load) - m_new) + gamma * (2 * d * (int(load[a]) - int(load[b]) - d))


def plan_swaps(counts, home: Sequence[int], G: int, E: int, tau: int = 0, gamma: Fraction = Fraction(0),
               max_swaps_per_rank: int = 1 << 30) -> Tuple[np.ndarray, List[Tuple[int, int]], np.ndarray]:
    """Returns (new home map, swaps as (e_a, e_b) in acceptance order, rank
    loads after the swaps).  Homes outside [0, G) read as rank 0."""
    n = [int(sum(int(counts[s][e]) for s in range(G))) for e in range(E)]
    where = [int(h) if 0 <= int(h) < G else 0 for h in home]
    load = [0] * G
    for e in range(E):
        load[where[e]] += n[e]
    budget = [max_swaps_per_rank] * G
    moved = [False] * E
    swaps: List[Tuple[int, int]] = []
    while True:
        a = max(range(G), key=lambda r: (load[r], -r))
        b = min(range(G), key=lambda r: (load[r], r))
        if load[a] - load[b] <= tau or budget[a] == 0 or budget[b] == 0:
            break
        best = None
        for ea in range(E):
            if where[ea] != a or moved[ea]:
                continue
            for eb in range(E):
                if where[eb] != b or moved[eb]:
                    continue
                gain = swap_benefit(load, a, b, n[ea], n[eb], gamma)
                if gain > 0 and (best is None or gain > best[0]):
                    best = (gain, ea, eb)  # first in (e_a, e_b) order wins ties
        if best is None:
            break
        _, ea, eb = best
        d = n[ea] - n[eb]
        load[a] -= d
        load[b] += d
        where[ea], where[eb] = b, a
        moved[ea] = moved[eb] = True
        budget[a] -= 1
        budget[b] -= 1
        swaps.append((ea, eb))
    return np.array(where, dtype=np.int32), swaps, np.array(load, dtype=np.int64)
