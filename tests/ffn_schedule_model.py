"""Model of the grouped FFN's schedule tables, for tests: the expert-major
virtual row order, its M tiles and the virtual -> physical row map, as the
schedule and row-map kernels define them (group g covers the clamped rows
[lo, hi), lo = clamp(group_off[g], 0, rows), hi = clamp(group_off[g+1], lo,
rows); unselected groups count as empty).  Plain loops over the definition;
the tests compare the device tables with it and check that every row a GEMM
tile reads lies inside the buffers, whatever the offsets hold."""
from __future__ import annotations

import numpy as np

SCHED_MIN_BM = 64


def clamp_range(group_off, g, rows):
    lo = min(max(int(group_off[g]), 0), rows)
    hi = min(max(int(group_off[g + 1]), lo), rows)
    return lo, hi


def schedule(group_off, num_groups, E, G, rank, rows, BM):
    """eoff[E+1], gvb[num_groups] (capped at rows), M tiles [(e, v0)]."""
    n = [0] * E
    gvb = [0] * num_groups
    for e in range(E):
        for g in range(e, num_groups, E):
            lo, hi = clamp_range(group_off, g, rows)
            if rank < 0 or (g // E) % G == rank:
                n[e] += hi - lo
    eoff = [0] * (E + 1)
    incl = 0
    for e in range(E):
        eoff[e] = min(incl, rows)
        incl += n[e]
    eoff[E] = min(incl, rows)
    tiles = []
    for e in range(E):
        run = eoff[e]
        for g in range(e, num_groups, E):
            lo, hi = clamp_range(group_off, g, rows)
            gvb[g] = min(run, rows)
            if rank < 0 or (g // E) % G == rank:
                run += hi - lo
        for v0 in range(eoff[e], eoff[e + 1], BM):
            tiles.append((e, v0))
    return eoff, gvb, tiles


def rowmap(group_off, num_groups, E, rows, eoff, gvb, gather=None, gather_k=1, rows_x=None):
    """rowmap[v] and asrc[v] for v < eoff[E]: expert = last e with eoff[e] <=
    v, group = last group g of e with gvb[g] <= v, row = lo_g + v - gvb[g]."""
    rows_x = rows if rows_x is None else rows_x
    nv = eoff[E]
    rm = np.zeros(nv, np.int64)
    src = np.zeros(nv, np.int64)
    for v in range(nv):
        e = max(i for i in range(E) if eoff[i] <= v)
        g = max(g for g in range(e, num_groups, E) if gvb[g] <= v)
        lo, _ = clamp_range(group_off, g, rows)
        q = min(max(lo + v - gvb[g], 0), rows - 1)
        rm[v] = q
        s = int(gather[q]) // gather_k if gather is not None else q
        src[v] = s if 0 <= s < rows_x else 0
    return rm, src


def max_mtiles(rows, E):
    return (rows + SCHED_MIN_BM - 1) // SCHED_MIN_BM + E


def workspace_offsets(rows, num_groups, E, inter, elem_bytes):
    """Byte offsets of the tables inside the FFN workspace (each table starts
    on a 256-byte boundary, in this order)."""
    al = lambda n: (n + 255) // 256 * 256  # noqa: E731
    mt = max_mtiles(rows, E)
    sizes = [("eoff", (E + 1) * 4), ("gvb", num_groups * 4), ("mt_e", mt * 4), ("mt_v0", mt * 4), ("n_mtiles", 4),
             ("rowmap", rows * 4), ("asrc", rows * 4), ("amid", rows * inter * elem_bytes)]
    off, out = 0, {}
    for name, n in sizes:
        out[name] = off
        off += al(n)
    out["total"] = off
    return out
