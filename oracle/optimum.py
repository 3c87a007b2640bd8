"""Exact optima that pin the plan and split heuristics (test infrastructure).

The per-step optimum of Relief ("The Per-Step Optimum Problem": minimise z
subject to every rank load L_i(x) <= z) is, for a fixed placement and whole
tokens, a transportation problem: each replicated expert's remote pool is
distributed over its hosts.  Its integer optimum is found here two ways --
exhaustive enumeration on tiny inputs, and binary search on z with a max-flow
feasibility test -- and the placement optimum by enumerating every placement
that gives each rank at most N non-resident experts.
"""
from __future__ import annotations

import itertools
from typing import List, Sequence

import numpy as np
from scipy.sparse import csr_matrix
from scipy.sparse.csgraph import maximum_flow

from .moe_oracle import host_sets


def _fixed_and_pools(c, home, hosts: List[set], G: int, E: int):
    f = [0] * G
    pools = []  # (R, sorted hosts) of experts whose pool can be split
    for e in range(E):
        R = sum(int(c[s][e]) for s in range(G) if s not in hosts[e])
        for s in hosts[e]:
            f[s] += int(c[s][e])
        if len(hosts[e]) == 1:
            f[int(home[e])] += R
        elif R > 0:
            pools.append((R, sorted(hosts[e])))
    return f, pools


def _compositions(R: int, m: int):
    if m == 1:
        yield (R,)
        return
    for a in range(R + 1):
        for rest in _compositions(R - a, m - 1):
            yield (a,) + rest


def split_optimum_bruteforce(c, home, replica, G: int, E: int) -> int:
    """min over every whole-token split of the max rank load (tiny inputs)."""
    hosts = host_sets(home, replica, E)
    f, pools = _fixed_and_pools(c, home, hosts, G, E)
    best = None
    for choice in itertools.product(*[list(_compositions(R, len(H))) for R, H in pools]):
        load = list(f)
        for (R, H), xs in zip(pools, choice):
            for h, x in zip(H, xs):
                load[h] += x
        m = max(load)
        best = m if best is None else min(best, m)
    return max(f) if best is None else best


def _feasible(z: int, f, pools, G: int) -> bool:
    if any(fi > z for fi in f):
        return False
    total = sum(R for R, _ in pools)
    if total == 0:
        return True
    P = len(pools)
    n = 2 + P + G           # 0 source, 1..P pools, P+1..P+G ranks, last sink
    src, sink = 0, n - 1
    rows, cols, caps = [], [], []
    for i, (R, H) in enumerate(pools):
        rows.append(src); cols.append(1 + i); caps.append(R)
        for h in H:
            rows.append(1 + i); cols.append(1 + P + h); caps.append(R)
    for r in range(G):
        rows.append(1 + P + r); cols.append(sink); caps.append(z - f[r])
    graph = csr_matrix((np.array(caps, dtype=np.int32), (rows, cols)), shape=(n, n))
    return maximum_flow(graph, src, sink).flow_value == total


def split_optimum(c, home, replica, G: int, E: int) -> int:
    """Integer per-step optimum of the max rank load for a fixed placement,
    by binary search on z with a max-flow feasibility check."""
    hosts = host_sets(home, replica, E)
    f, pools = _fixed_and_pools(c, home, hosts, G, E)
    lo = max(max(f), -(-(sum(f) + sum(R for R, _ in pools)) // G))
    hi = max(f) + sum(R for R, _ in pools)
    while lo < hi:
        mid = (lo + hi) // 2
        if _feasible(mid, f, pools, G):
            hi = mid
        else:
            lo = mid + 1
    return lo


def placement_optimum(c, home: Sequence[int], G: int, E: int, N: int) -> int:
    """min over every placement (each rank imports at most N non-resident
    experts) of the per-step split optimum (tiny inputs only)."""
    best = None
    per_rank = []
    for r in range(G):
        nonres = [e for e in range(E) if int(home[e]) != r]
        opts = []
        for n in range(N + 1):
            opts.extend(itertools.combinations(nonres, n))
        per_rank.append(opts)
    for choice in itertools.product(*per_rank):
        replica = np.full((G, max(N, 1)), -1, dtype=np.int32)
        for r, es in enumerate(choice):
            for i, e in enumerate(es):
                replica[r][i] = e
        v = split_optimum(c, home, replica, G, E)
        best = v if best is None else min(best, v)
    return best
