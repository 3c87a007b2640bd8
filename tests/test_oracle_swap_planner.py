"""Pins of FreeBalance's swap planner (oracle/swap_planner.py): the closed-form
benefit against eq. 8 evaluated directly, hand-worked plans, budgets and
thresholds, and invariants on random instances."""
from fractions import Fraction

import numpy as np

from oracle import swap_planner as S


def _counts_from_n(n, G):
    """A count matrix whose column sums are n (all pairs owned by rank 0)."""
    c = np.zeros((G, len(n)), np.int64)
    c[0] = n
    return c


def test_benefit_closed_form_equals_eq8():
    rng = np.random.default_rng(1)
    for _ in range(300):
        G = int(rng.integers(2, 7))
        load = [int(v) for v in rng.integers(0, 100, G)]
        a, b = (int(v) for v in rng.choice(G, 2, replace=False))
        na, nb = int(rng.integers(0, 40)), int(rng.integers(0, 40))
        gamma = Fraction(int(rng.integers(0, 5)), int(rng.integers(1, 4)))
        new = list(load)
        new[a] += nb - na
        new[b] += na - nb
        assert S.swap_benefit(load, a, b, na, nb, gamma) == S.phi(load, gamma) - S.phi(new, gamma)


def test_two_rank_plan_by_hand():
    # L = [16, 4]; gamma = 0: benefits 3, 5, 5, 3 -> (e0, e3) by the
    # lower e_a; then the only candidate (e2, e1) would raise the max
    home = [0, 0, 1, 1]
    c = _counts_from_n([10, 6, 1, 3], 2)
    for gamma in (Fraction(0), Fraction(1)):
        where, swaps, load = S.plan_swaps(c, home, 2, 4, gamma=gamma)
        assert where.tolist() == [1, 0, 1, 0] and swaps == [(0, 3)] and load.tolist() == [9, 11]


def test_variance_term_moves_past_a_tied_straggler():
    # ranks 0 and 1 both at 20: no swap between 0 and 2 lowers the max, so
    # gamma = 0 plans nothing; gamma = 1 swaps (e0, e4), then (e2, e1)
    home = [0, 0, 1, 1, 2, 2]
    c = _counts_from_n([12, 8, 15, 5, 1, 1], 3)
    where, swaps, load = S.plan_swaps(c, home, 3, 6, gamma=Fraction(0))
    assert swaps == [] and load.tolist() == [20, 20, 2]
    where, swaps, load = S.plan_swaps(c, home, 3, 6, gamma=Fraction(1))
    assert swaps == [(0, 4), (2, 1)] and where.tolist() == [2, 1, 0, 1, 0, 2] and load.tolist() == [16, 13, 13]
    # one swap per rank: rank 0's budget is spent by the first swap
    _, swaps, load = S.plan_swaps(c, home, 3, 6, gamma=Fraction(1), max_swaps_per_rank=1)
    assert swaps == [(0, 4)] and load.tolist() == [9, 20, 13]
    # threshold: after the first swap the gap is 20 - 9 = 11
    _, swaps, _ = S.plan_swaps(c, home, 3, 6, gamma=Fraction(1), tau=11)
    assert swaps == [(0, 4)]


def test_plan_invariants():
    rng = np.random.default_rng(4)
    for _ in range(60):
        G = int(rng.choice([2, 3, 4, 8]))
        E = G * int(rng.choice([1, 2, 4]))
        pop = 1.0 / (1 + rng.permutation(E)) ** rng.uniform(0.3, 1.5)
        c = np.stack([rng.multinomial(int(rng.integers(0, 500)), pop / pop.sum()) for _ in range(G)])
        home = rng.permutation(np.arange(E) // (E // G)).astype(np.int32)
        gamma = Fraction(int(rng.integers(0, 3)), int(rng.integers(1, 1000)))
        budget = int(rng.choice([1, 2, 100]))
        tau = int(rng.choice([0, 5]))
        where, swaps, load = S.plan_swaps(c, home, G, E, tau=tau, gamma=gamma, max_swaps_per_rank=budget)
        n = c.sum(axis=0)
        assert np.bincount(where, minlength=G).tolist() == np.bincount(home, minlength=G).tolist()
        assert np.array_equal(load, np.bincount(where, weights=n, minlength=G).astype(np.int64))
        flat = [e for s in swaps for e in s]
        assert len(flat) == len(set(flat))  # an expert moves at most once
        # replay: every accepted swap lowers eq. 8 and stays within budget
        cur = list(home)
        L = np.bincount(cur, weights=n, minlength=G).astype(np.int64).tolist()
        used = [0] * G
        for ea, eb in swaps:
            a, b = cur[ea], cur[eb]
            new = list(L)
            new[a] += int(n[eb]) - int(n[ea])
            new[b] += int(n[ea]) - int(n[eb])
            assert S.phi(new, gamma) < S.phi(L, gamma)
            assert max(L) - min(L) > tau
            # the frontier: most-loaded rank to least-loaded rank, lower index on ties
            assert a == max(range(G), key=lambda r: (L[r], -r)) and b == min(range(G), key=lambda r: (L[r], r))
            cur[ea], cur[eb] = b, a
            used[a] += 1
            used[b] += 1
            L = new
        assert max(used) <= budget
        assert cur == where.tolist()
