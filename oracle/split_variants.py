"""Alternative per-step splits of the remote pools, and the stale-split
measurement (test infrastructure only, like the rest of ``oracle/``).

Sources:

* Relief ("A Per-Step Load-Balancing Engine for Expert-Parallel MoE
  Serving"), "Ablation Results (Table III)": the engine without its reverse
  move, with snapshot (Jacobi) loads and damping, with water-filling or
  proportional relaxation in place of pairwise halving, and the hash split;
  "Failure of Existing Approaches" (decision frequency: a split reused one
  step later).
* Libra README, "Key Ideas" (adaptive token sharding): remote tokens move
  from overloaded GPUs to the least-loaded GPU that holds a replica of their
  expert.

The pages name these variants without their exact rules; the reading taken
for each is stated at its function.  Common to all: whole tokens; a host of
e serves its own tokens of e; an unreplicated expert's remote pool goes to
its home; a replicated expert's pool starts from the even split over its
hosts (ascending rank), except Libra's sharding, which starts with every pool
on its home.  Transfers and rounds are those of ``moe_oracle.split``.
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import Dict, Sequence, Tuple

import numpy as np

from .moe_oracle import _remote_pool, colour_transfers, even_split, host_sets, signed_move, split, split_transfers

VARIANTS = ("relief", "no_reverse", "jacobi", "water_fill", "proportional", "hash", "libra_greedy")


def _start(c, home, hosts, G: int, E: int, pools_at_home: bool):
    """Fixed loads plus the starting placement of every pool; x[e][h] is the
    mass of e's pool on host h for replicated experts."""
    load = [0] * G
    x: Dict[int, Dict[int, int]] = {}
    fixed_host = {}
    for e in range(E):
        R = _remote_pool(c, hosts[e], e, G)
        for s in hosts[e]:
            load[s] += int(c[s][e])
        if len(hosts[e]) == 1:
            h = int(home[e])
            load[h] += R
            fixed_host[e] = (h, R)
        else:
            Hs = sorted(hosts[e])
            x[e] = {h: 0 for h in Hs}
            if pools_at_home:
                x[e][int(home[e])] = R
            else:
                x[e] = even_split(R, Hs)
            for h, m in x[e].items():
                load[h] += m
    return load, x, fixed_host


def _result(x, fixed_host, load, G: int, E: int):
    host_count = np.zeros((E, G), dtype=np.int64)
    for e, (h, R) in fixed_host.items():
        host_count[e][h] = R
    for e, xe in x.items():
        for h, m in xe.items():
            host_count[e][h] = m
    return host_count, np.array(load, dtype=np.int64)


def _rounds(home, hosts, E: int):
    transfers = split_transfers(home, hosts, E)
    colours = colour_transfers(transfers)
    n = (max(colours) + 1) if colours else 0
    return [[t for t, col in zip(transfers, colours) if col == r] for r in range(n)], len(transfers)


def _pairwise(c, home, replica, G: int, E: int, passes: int, eps: int, reverse: bool, snapshot: bool):
    """Relief's pairwise relaxation with one ingredient changed.

    reverse=False (reading of "without reverse move"): a transfer (u = home,
    v = replica) only moves mass from u to v, when u is the heavier side.
    snapshot=True (reading of "snapshot loads, damped (Jacobi)"): every
    transfer of a pass reads the loads as they were when the pass began, and
    moves a quarter of that gap (the half-gap move damped by one more
    halving, since a rank in several transfers receives several moves), still
    capped by the giver's current mass."""
    hosts = host_sets(home, replica, E)
    load, x, fixed_host = _start(c, home, hosts, G, E, pools_at_home=False)
    rounds, _ = _rounds(home, hosts, E)
    for _p in range(passes):
        snap = list(load)
        moved = False
        for rnd in rounds:
            for (u, v, e) in rnd:
                gap = (snap[u] - snap[v]) if snapshot else (load[u] - load[v])
                if gap <= 0 and not reverse:
                    continue
                f = signed_move(gap, 2 if snapshot else 1, x[e][u], x[e][v])
                if abs(f) > eps:
                    load[u] -= f
                    load[v] += f
                    x[e][u] -= f
                    x[e][v] += f
                    moved = True
        if not moved:
            break
    return _result(x, fixed_host, load, G, E)


def water_fill_pool(R: int, levels: Sequence[Tuple[int, int]]) -> Dict[int, int]:
    """Integer water-filling of R tokens over hosts given as (rank, load):
    the largest level z with sum(max(0, z - load)) <= R is filled, and the
    tokens left over (fewer than the hosts at or below z) go one each to
    those hosts in ascending rank."""
    loads = [l for _, l in levels]
    lo, hi = min(loads), min(loads) + R  # z = hi is always affordable only if one host
    while lo < hi:  # largest affordable z
        mid = (lo + hi + 1) // 2
        if sum(max(0, mid - l) for l in loads) <= R:
            lo = mid
        else:
            hi = mid - 1
    z = lo
    give = {r: max(0, z - l) for r, l in levels}
    left = R - sum(give.values())
    for r, l in sorted(levels):
        if left == 0:
            break
        if l <= z:
            give[r] += 1
            left -= 1
    return give


def proportional_pool(R: int, levels: Sequence[Tuple[int, int]]) -> Dict[int, int]:
    """R tokens over hosts (rank, load) in proportion to 1 / (load + 1); whole
    tokens by largest remainder, ties to the lower rank."""
    wts = {r: Fraction(1, l + 1) for r, l in levels}
    tot = sum(wts.values())
    exact = {r: R * w / tot for r, w in wts.items()}
    give = {r: math.floor(v) for r, v in exact.items()}
    left = R - sum(give.values())
    for r in sorted(exact, key=lambda r: (-(exact[r] - give[r]), r))[:left]:
        give[r] += 1
    return give


def _per_expert(c, home, replica, G: int, E: int, passes: int, rule):
    """Reading of the water-filling and proportional relaxations (named in the
    ablation table without their rules): each pass, every replicated expert
    redistributes its whole pool by ``rule`` over its hosts' loads as they were
    when the pass began, less its own mass there -- all pools at once, from one
    snapshot, as the standard relaxations run (Relief's own move is pairwise
    and reads the loads its round before left).  Stops after a pass that
    changes nothing."""
    hosts = host_sets(home, replica, E)
    load, x, fixed_host = _start(c, home, hosts, G, E, pools_at_home=False)
    for _p in range(passes):
        snap = list(load)
        new = {e: rule(sum(xe.values()), [(h, snap[h] - xe[h]) for h in sorted(xe)]) for e, xe in x.items()}
        if new == x:
            break
        for e, xe in x.items():
            for h in xe:
                load[h] += new[e][h] - xe[h]
        x = new
    return _result(x, fixed_host, load, G, E)


def libra_greedy(c, home, replica, G: int, E: int, passes: int = 12):
    """Reading of Libra's adaptive token sharding: every remote pool starts on
    its home.  Repeatedly take the most-loaded rank a (ties: lower rank); walk
    the replicated experts with mass on a by that mass descending (ties: lower
    id); for each, b is its least-loaded other host (ties: lower rank); the
    first with load[a] - load[b] >= 2 moves min(mass on a, (load[a] -
    load[b]) >> 1) tokens from a to b.  Stops when no expert of a can move,
    or after passes x (number of replica transfers) moves."""
    hosts = host_sets(home, replica, E)
    load, x, fixed_host = _start(c, home, hosts, G, E, pools_at_home=True)
    n_transfers = sum(len(hs) - 1 for hs in hosts)
    for _m in range(passes * max(1, n_transfers)):
        a = max(range(G), key=lambda r: (load[r], -r))
        cand = sorted((e for e in x if x[e].get(a, 0) > 0), key=lambda e: (-x[e][a], e))
        move = None
        for e in cand:
            b = min((h for h in x[e] if h != a), key=lambda r: (load[r], r))
            if load[a] - load[b] >= 2:
                move = (e, b, min(x[e][a], (load[a] - load[b]) >> 1))
                break
        if move is None:
            break
        e, b, d = move
        load[a] -= d
        load[b] += d
        x[e][a] -= d
        x[e][b] += d
    return _result(x, fixed_host, load, G, E)


def split_variant(c, home, replica, G: int, E: int, variant: str, passes: int = 12, eps: int = 0):
    """host_count[E][G] and load[G] of one split variant (see VARIANTS)."""
    if variant == "relief":
        return split(c, home, replica, G, E, passes=passes, eps=eps)
    if variant == "hash":
        return split(c, home, replica, G, E, passes=0)
    if variant == "no_reverse":
        return _pairwise(c, home, replica, G, E, passes, eps, reverse=False, snapshot=False)
    if variant == "jacobi":
        return _pairwise(c, home, replica, G, E, passes, eps, reverse=True, snapshot=True)
    if variant == "water_fill":
        return _per_expert(c, home, replica, G, E, passes, water_fill_pool)
    if variant == "proportional":
        return _per_expert(c, home, replica, G, E, passes, proportional_pool)
    if variant == "libra_greedy":
        return libra_greedy(c, home, replica, G, E, passes)
    raise ValueError(variant)


def stale_split(c, home, replica, host_count_prev, G: int, E: int):
    """The split of an earlier step reused (Relief, "Failure of Existing
    Approaches", decision frequency).  Reading: same placement; each
    replicated expert's new remote pool R is dealt in the fractions
    host_count_prev[e][h] / (sum of host_count_prev[e] over e's current
    hosts; negative entries read as 0), whole tokens by largest remainder
    (ties: lower rank); an expert whose earlier pool on its hosts was empty
    deals evenly; an unreplicated expert keeps its whole pool at home.  Returns (host_count[E][G], load[G])
    in the split's conventions."""
    hosts = host_sets(home, replica, E)
    load = [0] * G
    host_count = np.zeros((E, G), dtype=np.int64)
    for e in range(E):
        R = _remote_pool(c, hosts[e], e, G)
        for s in hosts[e]:
            load[s] += int(c[s][e])
        Hs = sorted(hosts[e])
        if len(Hs) == 1:
            give = {Hs[0]: R}
        else:
            prev = {h: max(0, int(host_count_prev[e][h])) for h in Hs}
            tot = sum(prev.values())
            if tot == 0:
                give = even_split(R, Hs)
            else:
                give = {h: (R * prev[h]) // tot for h in Hs}
                rem = {h: (R * prev[h]) % tot for h in Hs}
                left = R - sum(give.values())
                for h in sorted(Hs, key=lambda h: (-rem[h], h))[:left]:
                    give[h] += 1
        for h, m in give.items():
            load[h] += m
            host_count[e][h] = m
    return host_count, np.array(load, dtype=np.int64)


def stale_loads(c, home, replica, host_count_prev, G: int, E: int) -> np.ndarray:
    """Rank loads of ``stale_split``."""
    return stale_split(c, home, replica, host_count_prev, G, E)[1]
