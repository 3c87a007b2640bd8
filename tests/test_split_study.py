"""Balance attained by the split variants, and what a stale split costs
(oracle only; the GPU variants equal their oracles bit for bit, see
test_gpu_parity.py).  Run with ``-s`` to print the tables.

Attainment = per-step optimum of the max rank load (max-flow, for the same
placement and counts) / the max rank load the variant leaves -- Relief's
"Convergence and Pass Count" and Table III measure the same ratio.
Instances: Zipf(1.2) expert popularity; the plan (N = 4 slots, L = 2
locality imports) is made from a predicted count matrix and the split runs
on the actual one, each popularity perturbed by its own log-normal factor
(sigma 0.3); 8192 pairs per rank.
"""
import numpy as np

from oracle import moe_oracle as O
from oracle import split_variants as V
from oracle.optimum import split_optimum


def _drift_instance(rng, G, E, N=4, pairs=8192, sigma=0.3, zipf=1.2):
    pop = 1.0 / (1 + rng.permutation(E)) ** zipf
    pred = pop * np.exp(rng.normal(0, sigma, E))
    act = pop * np.exp(rng.normal(0, sigma, E))
    cp = np.stack([rng.multinomial(pairs, pred / pred.sum()) for _ in range(G)])
    c = np.stack([rng.multinomial(pairs, act / act.sum()) for _ in range(G)])
    home = (np.arange(E) // (E // G)).astype(np.int32)
    return c, home, O.plan(cp, home, G, E, N, N // 2)


def test_variant_attainment():
    rng = np.random.default_rng(2026)
    table = {}
    for G, E in ((16, 128), (64, 256)):
        att = {v: [] for v in V.VARIANTS + ("static",)}
        for _ in range(6):
            c, home, rep = _drift_instance(rng, G, E)
            opt = split_optimum(c, home, rep, G, E)
            for v in V.VARIANTS:
                _, ld = V.split_variant(c, home, rep, G, E, v)
                att[v].append(opt / ld.max())
            att["static"].append(opt / max(O.static_loads(c, home, G, E)))
        table[G] = {v: 100 * float(np.mean(a)) for v, a in att.items()}
    print("\nattainment of the per-step optimum, % (mean of 6 instances)")
    print("variant        " + "".join(f"G={G:<8}" for G in table))
    for v in V.VARIANTS + ("static",):
        print(f"{v:<15}" + "".join(f"{table[G][v]:<10.2f}" for G in table))
    for G, row in table.items():
        assert row["relief"] >= 99.0, G
        assert all(row["relief"] >= row[v] for v in V.VARIANTS), G


def test_stale_split_loss():
    """Decision frequency (Relief, "Failure of Existing Approaches"): the
    split made for step s dealt again at step s+1.  Reading: the placement
    (planned from step s's counts) stays; step s+1's popularity is step s's
    times a log-normal factor of the given sigma.  Loss = (stale - fresh) /
    (baseline - fresh) in max rank load, the part of the fresh split's gain
    that reuse gives up, against two baselines: the even split on the same
    placement, and no balancing at all (every pair at its home)."""
    rng = np.random.default_rng(7)
    G, E, N = 16, 128, 4
    print("\nstale split: loss of the fresh split's gain, % (mean of 6 step pairs)")
    print("sigma   vs even split   vs no balancing")
    res = {}
    for sigma in (0.1, 0.3, 1.0):
        l_even, l_static = [], []
        while len(l_even) < 6:
            pop = 1.0 / (1 + rng.permutation(E)) ** 1.2
            pop1 = pop * np.exp(rng.normal(0, sigma, E))
            c0 = np.stack([rng.multinomial(8192, pop / pop.sum()) for _ in range(G)])
            c1 = np.stack([rng.multinomial(8192, pop1 / pop1.sum()) for _ in range(G)])
            home = (np.arange(E) // (E // G)).astype(np.int32)
            rep = O.plan(c0, home, G, E, N, N // 2)
            hc0, _ = O.split(c0, home, rep, G, E)
            _, fresh = O.split(c1, home, rep, G, E)
            _, even = O.split(c1, home, rep, G, E, passes=0)
            static = max(O.static_loads(c1, home, G, E))
            stale = V.stale_loads(c1, home, rep, hc0, G, E)
            if even.max() > fresh.max():
                l_even.append((stale.max() - fresh.max()) / (even.max() - fresh.max()))
                l_static.append((stale.max() - fresh.max()) / (static - fresh.max()))
        res[sigma] = (float(np.mean(l_even)), float(np.mean(l_static)))
        print(f"{sigma:<8}{100 * res[sigma][0]:<16.1f}{100 * res[sigma][1]:.1f}")
    assert all(e > 0 and st > 0 for e, st in res.values())
    assert res[1.0][1] > res[0.1][1]
