"""Pins of the split variants and the stale-split loads (oracle/split_variants.py):
hand-worked small cases, closed forms, the max-flow optimum, invariants."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from oracle import split_variants as V
from oracle.optimum import split_optimum


def _three_rank_two_pools(R):
    """Experts 0 and 1 live on rank 0; rank 1 replicates e0, rank 2 replicates
    e1.  Rank 0 holds 60 own tokens of e0; rank 2 sends R tokens of e0 and
    rank 1 sends R tokens of e1 (the two remote pools).  Loads after the even
    split: [60 + R, R/2, R/2]."""
    G, E = 3, 3
    home = np.array([0, 0, 2], np.int32)
    rep = np.array([[-1], [0], [1]], np.int32)
    c = np.zeros((G, E), np.int64)
    c[0][0] = 60
    c[2][0] = R
    c[1][1] = R
    return c, home, rep, G, E


def _two_host_pool(heavy_replica):
    """e0 on rank 0, replicated on rank 1; rank 2 sends 10 tokens of e0 (even
    split 5/5).  Rank 1 also serves 20 tokens of its own expert e1 when
    heavy_replica, else rank 0 serves 20 of e0 itself."""
    G, E = 3, 3
    home = np.array([0, 1, 2], np.int32)
    rep = np.array([[-1], [0], [-1]], np.int32)
    c = np.zeros((G, E), np.int64)
    c[2][0] = 10
    if heavy_replica:
        c[1][1] = 20
    else:
        c[0][0] = 20
    return c, home, rep, G, E


def test_hash_is_the_even_split():
    c, home, rep, G, E = _three_rank_two_pools(200)
    hc, ld = V.split_variant(c, home, rep, G, E, "hash")
    assert hc[0].tolist() == [100, 100, 0] and hc[1].tolist() == [100, 0, 100]
    assert ld.tolist() == [260, 100, 100]


def test_no_reverse_keeps_mass_off_the_home_only():
    # replica heavier: Relief moves 5 back to the home (gap -20, capped by the
    # replica's mass 5); without the reverse move nothing moves
    c, home, rep, G, E = _two_host_pool(heavy_replica=True)
    hc, ld = V.split_variant(c, home, rep, G, E, "relief")
    assert ld.tolist() == [10, 20, 0] and hc[0].tolist() == [10, 0, 0]
    hc, ld = V.split_variant(c, home, rep, G, E, "no_reverse")
    assert ld.tolist() == [5, 25, 0] and hc[0].tolist() == [5, 5, 0]
    # home heavier (25 vs 5): both move half the gap, 10, capped by the home's mass 5
    c, home, rep, G, E = _two_host_pool(heavy_replica=False)
    for v in ("relief", "no_reverse"):
        hc, ld = V.split_variant(c, home, rep, G, E, v)
        assert ld.tolist() == [20, 10, 0] and hc[0].tolist() == [0, 10, 0], v


def test_relief_and_jacobi_by_hand():
    c, home, rep, G, E = _three_rank_two_pools(200)
    # Relief, one pass: round 0 (0,1): gap 160 -> 80; round 1 (0,2) reads
    # the new load 180: gap 80 -> 40
    hc, ld = V.split_variant(c, home, rep, G, E, "relief", passes=1)
    assert ld.tolist() == [140, 180, 140]
    # Jacobi, one pass: both transfers read the snapshot [260,100,100] and
    # move a quarter of 160
    hc, ld = V.split_variant(c, home, rep, G, E, "jacobi", passes=1)
    assert ld.tolist() == [180, 140, 140] and hc[0].tolist() == [60, 140, 0]
    # to the end (worked pass by pass): Relief 153/154/153, Jacobi 154/153/153
    _, ld = V.split_variant(c, home, rep, G, E, "relief")
    assert ld.tolist() == [153, 154, 153]
    hc, ld = V.split_variant(c, home, rep, G, E, "jacobi")
    assert ld.tolist() == [154, 153, 153] and hc[0].tolist() == [47, 153, 0] and hc[1].tolist() == [47, 0, 153]


def test_water_fill_pool_closed_form():
    assert V.water_fill_pool(12, [(0, 10), (1, 0), (2, 4)]) == {0: 0, 1: 8, 2: 4}  # level 8
    assert V.water_fill_pool(5, [(0, 0), (1, 0)]) == {0: 3, 1: 2}  # level 2, one left to the lower rank
    assert V.water_fill_pool(0, [(3, 7), (5, 1)]) == {3: 0, 5: 0}
    assert V.water_fill_pool(7, [(4, 2)]) == {4: 7}


def test_proportional_pool_closed_form():
    # weights 1 and 1/2: exact 20/3 and 10/3 -> 6 and 3, the remaining token
    # to the larger remainder
    assert V.proportional_pool(10, [(0, 0), (1, 1)]) == {0: 7, 1: 3}
    assert V.proportional_pool(9, [(2, 5), (7, 5), (9, 5)]) == {2: 3, 7: 3, 9: 3}
    assert V.proportional_pool(1, [(2, 5), (7, 5)]) == {2: 1, 7: 0}


def test_water_fill_is_optimal_for_a_single_pool():
    # one replicated expert: filling its hosts to a common level minimises the
    # max load (checked against the max-flow optimum)
    rng = np.random.default_rng(3)
    for _ in range(20):
        G, E = 6, 6
        home = np.arange(E, dtype=np.int32)
        rep = np.full((G, 1), -1, np.int32)
        hosts = rng.choice(np.arange(1, G), size=int(rng.integers(1, 4)), replace=False)
        rep[hosts, 0] = 0
        c = rng.integers(0, 30, (G, E))
        _, ld = V.split_variant(c, home, rep, G, E, "water_fill")
        assert ld.max() == split_optimum(c, home, rep, G, E)


def test_libra_greedy_by_hand():
    # pool of 10 starts on the home (load 10 vs 2): one move of 4, then
    # a tie at 6 that no move improves
    G, E = 3, 3
    home = np.array([0, 1, 2], np.int32)
    rep = np.array([[-1], [0], [-1]], np.int32)
    c = np.zeros((G, E), np.int64)
    c[2][0] = 10
    c[1][1] = 2
    hc, ld = V.split_variant(c, home, rep, G, E, "libra_greedy")
    assert ld.tolist() == [6, 6, 0] and hc[0].tolist() == [6, 4, 0]


def _random_instance(rng, G, E, N):
    pop = 1.0 / (1 + rng.permutation(E)) ** rng.uniform(0.6, 1.5)
    c = np.stack([rng.multinomial(int(rng.integers(0, 600)), pop / pop.sum()) for _ in range(G)]).astype(np.int64)
    home = (np.arange(E) // (E // G)).astype(np.int32)
    rep = O.plan(c, home, G, E, N, N // 2) if N else None
    return c, home, rep


@pytest.mark.parametrize("variant", V.VARIANTS)
def test_variant_invariants(variant):
    rng = np.random.default_rng(7)
    for _ in range(25):
        G = int(rng.choice([2, 3, 4, 8]))
        E = G * int(rng.choice([1, 2, 4]))
        N = int(rng.integers(0, 3))
        c, home, rep = _random_instance(rng, G, E, N)
        hc, ld = V.split_variant(c, home, rep, G, E, variant)
        hosts = O.host_sets(home, rep, E)
        fixed = np.zeros(G, np.int64)
        for e in range(E):
            pool = sum(int(c[s][e]) for s in range(G) if s not in hosts[e])
            assert hc[e].sum() == pool
            for r in range(G):
                if r in hosts[e]:
                    fixed[r] += c[r][e]
                else:
                    assert hc[e][r] == 0
        assert np.array_equal(ld, fixed + hc.sum(axis=0))
        assert ld.max() >= split_optimum(c, home, rep, G, E)
        if variant == "libra_greedy":
            # stopping rule: the most-loaded rank cannot hand tokens of any of
            # its replicated experts to a host at least 2 below it
            a = max(range(G), key=lambda r: (ld[r], -r))
            for e in range(E):
                if len(hosts[e]) > 1 and hc[e][a] > 0:
                    assert all(ld[a] - ld[b] < 2 for b in hosts[e] if b != a)


def test_stale_loads_reduce_to_the_split():
    rng = np.random.default_rng(9)
    for _ in range(10):
        G, E, N = 4, 8, 2
        c, home, rep = _random_instance(rng, G, E, N)
        hc, ld = O.split(c, home, rep, G, E)
        # the same step's fractions reproduce its loads; on doubled counts,
        # exactly doubled shares
        assert np.array_equal(V.stale_loads(c, home, rep, hc, G, E), ld)
        assert np.array_equal(V.stale_loads(2 * c, home, rep, hc, G, E), 2 * ld)
        hc2, ld2 = V.stale_split(c, home, rep, hc, G, E)
        assert np.array_equal(hc2, hc) and np.array_equal(ld2, ld)


def test_stale_split_by_hand():
    # expert 0 lives on rank 0 with replicas on ranks 1 and 2; its remote
    # pool is rank 3's pairs.  Expert 1 (home 1, no replica) gets rank 0's 4.
    G, E = 4, 4
    home = np.arange(4, dtype=np.int32)
    rep = np.array([[-1], [0], [0], [-1]], dtype=np.int32)
    c = np.zeros((G, E), np.int64)
    c[0][0], c[2][0], c[3][0], c[0][1] = 1, 2, 10, 4
    prev = np.zeros((E, G), np.int64)
    prev[0] = [1, 2, 0, 5]  # rank 3 is no host of expert 0: ignored
    hc, ld = V.stale_split(c, home, rep, prev, G, E)
    # 10 * (1, 2, 0) / 3 = (3, 6, 0) rem (1, 2, 0): the one left goes to rank 1
    assert hc[0].tolist() == [3, 7, 0, 0] and hc[1].tolist() == [0, 4, 0, 0]
    assert ld.tolist() == [1 + 3, 7 + 4, 2, 0]
    # equal remainders go to the lower ranks
    c[3][0] = 5
    prev[0] = [1, 1, 1, 0]
    assert V.stale_split(c, home, rep, prev, G, E)[0][0].tolist() == [2, 2, 1, 0]
    # no earlier pool on the current hosts: the even split
    prev[0] = [0, 0, 0, 9]
    assert V.stale_split(c, home, rep, prev, G, E)[0][0].tolist() == [2, 2, 1, 0]
    c[3][0] = 7
    assert V.stale_split(c, home, rep, prev, G, E)[0][0].tolist() == [3, 2, 2, 0]
    # negative entries read as 0: 7 * (0, 1, 1) / 2 = (0, 3, 3) rem (0, 1, 1)
    prev[0] = [-4, 1, 1, 0]
    assert V.stale_split(c, home, rep, prev, G, E)[0][0].tolist() == [0, 4, 3, 0]


def _two_pools_sharing_a_host():
    """Three ranks, one expert each (home = rank).  Rank 0 replicates e1 and
    e2, so e1's pool (its pairs owned by rank 2: 8) spreads over {0, 1} and
    e2's pool (its pairs owned by rank 1: 8) over {0, 2}; both pools share
    host 0.  Own tokens: rank 1 serves 10 of e1, rank 2 serves 10 of e2, rank
    0 none.  Even split 4/4 and 4/4: loads [8, 14, 14]."""
    G, E = 3, 3
    home = np.array([0, 1, 2], np.int32)
    rep = np.array([[1, 2], [-1, -1], [-1, -1]], np.int32)
    c = np.array([[0, 0, 0],
                  [0, 10, 8],
                  [0, 8, 10]], np.int64)
    return c, home, rep, G, E


def test_water_fill_two_pools_by_hand_snapshot_not_sequential():
    # Pass 1 reads the snapshot [8, 14, 14].  Levels (load less own mass):
    # e1: host 0 at 4, host 1 at 10; filling R = 8 reaches z = 11 exactly
    # ((11-4) + (11-10) = 8), so e1 -> {0: 7, 1: 1}; e2 the same over {0, 2}.
    # Loads [14, 11, 11].  (Sequential filling would let e2 see e1's move:
    # after e1, loads [11, 11, 14]; e2's levels 7 and 10 give z = 12 plus one
    # token to host 0 -> {0: 6, 2: 2}, loads [13, 11, 12].)
    c, home, rep, G, E = _two_pools_sharing_a_host()
    hc, ld = V.split_variant(c, home, rep, G, E, "water_fill", passes=1)
    assert ld.tolist() == [14, 11, 11]
    assert hc[1].tolist() == [7, 1, 0] and hc[2].tolist() == [7, 0, 1]
    # Pass 2 from [14, 11, 11]: levels 14-7 = 7 and 11-1 = 10; z = 12 takes
    # 5 + 2 = 7, the token left goes to host 0 (level 7 <= 12, lowest rank):
    # {0: 6, 1: 2}, e2 the same; loads [12, 12, 12].  Pass 3 reproduces it
    # (levels 6 and 10, z = 12 takes exactly 8) and the loop stops.
    hc, ld = V.split_variant(c, home, rep, G, E, "water_fill", passes=2)
    assert ld.tolist() == [12, 12, 12]
    assert hc[1].tolist() == [6, 2, 0] and hc[2].tolist() == [6, 0, 2]
    hc12, ld12 = V.split_variant(c, home, rep, G, E, "water_fill", passes=12)
    assert np.array_equal(hc12, hc) and np.array_equal(ld12, ld)


def test_proportional_two_pools_by_hand():
    # Pass 1, snapshot [8, 14, 14]: e1's levels 4 and 10 give weights 1/5 and
    # 1/11, shares 8*11/16 = 5.5 and 8*5/16 = 2.5; floors 5 and 2, the tied
    # remainder goes to the lower rank: {0: 6, 1: 2}; e2 the same.  Loads
    # [12, 12, 12].  (Sequential: e1 first gives loads [10, 12, 14], then e2's
    # levels 6 and 10 give 8*11/18 and 8*7/18 -> {0: 5, 2: 3}, loads
    # [11, 12, 13].)
    c, home, rep, G, E = _two_pools_sharing_a_host()
    hc, ld = V.split_variant(c, home, rep, G, E, "proportional", passes=1)
    assert ld.tolist() == [12, 12, 12]
    assert hc[1].tolist() == [6, 2, 0] and hc[2].tolist() == [6, 0, 2]
    # Pass 2 from [12, 12, 12]: levels 12-6 = 6 and 12-2 = 10, weights 1/7 and
    # 1/11: 88/18 = 4.89 and 56/18 = 3.11 -> floors 4 and 3, the larger
    # remainder (0.89) to host 0: {0: 5, 1: 3}; loads [10, 13, 13].
    hc, ld = V.split_variant(c, home, rep, G, E, "proportional", passes=2)
    assert ld.tolist() == [10, 13, 13]
    assert hc[1].tolist() == [5, 3, 0] and hc[2].tolist() == [5, 0, 3]
    # Pass 3 from [10, 13, 13]: levels 5 and 10, weights 1/6 and 1/11: 88/17 =
    # 5.18 and 48/17 = 2.82 -> floors 5 and 2, the larger remainder (0.82) to
    # host 1: {0: 5, 1: 3} again, so the loop stops there.
    hc12, ld12 = V.split_variant(c, home, rep, G, E, "proportional", passes=12)
    assert np.array_equal(hc12, hc) and np.array_equal(ld12, ld)
