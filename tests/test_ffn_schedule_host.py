"""The grouped FFN's schedule on any device offsets (CPU): every virtual row a
GEMM tile reads has a row-map entry, and every row it reads or writes lies in
[0, rows), also for offsets that decrease, overlap or leave [0, rows]."""
import numpy as np
from hypothesis import given, settings, strategies as st

from tests import ffn_schedule_model as F


def _check(group_off, num_groups, E, G, rank, rows, BM, gather=None, gather_k=1, rows_x=None):
    eoff, gvb, tiles = F.schedule(group_off, num_groups, E, G, rank, rows, BM)
    assert eoff[0] == 0 and all(a <= b for a, b in zip(eoff, eoff[1:])) and eoff[E] <= rows
    assert len(tiles) <= (rows + BM - 1) // BM + E  # at most one partial tile per expert
    if BM >= F.SCHED_MIN_BM:
        assert len(tiles) <= F.max_mtiles(rows, E)  # the tile tables' size
    rm, src = F.rowmap(group_off, num_groups, E, rows, eoff, gvb, gather, gather_k, rows_x)
    for e, v0 in tiles:
        vend = eoff[e + 1]
        assert eoff[e] <= v0 < vend <= eoff[E]
        # a tile reads rows [v0, min(v0 + BM, vend)) and redirects the rest to v0
        for v in range(v0, min(v0 + BM, vend)):
            assert 0 <= rm[v] < rows and 0 <= src[v] < (rows if rows_x is None else rows_x)
    # every virtual row lies in its group's clamped range
    for v in range(eoff[E]):
        e = max(i for i in range(E) if eoff[i] <= v)
        g = max(g for g in range(e, num_groups, E) if gvb[g] <= v)
        lo, hi = F.clamp_range(group_off, g, rows)
        assert lo <= rm[v] < hi
    return eoff, gvb, rm


def test_monotone_offsets_map_every_selected_row_once():
    rows, E, G = 40, 3, 2
    group_off = np.array([0, 5, 5, 9, 20, 21, 26, 27, 30, 31, 35, 40, 40])  # 2*G*E groups
    for rank in (-1, 0, 1):
        eoff, gvb, rm = _check(group_off, 2 * G * E, E, G, rank, rows, 8)
        want = sorted(q for g in range(2 * G * E) if rank < 0 or (g // E) % G == rank
                      for q in range(*F.clamp_range(group_off, g, rows)))
        assert sorted(rm.tolist()) == want


def test_decreasing_overlapping_and_out_of_range_offsets_stay_in_bounds():
    rows, E, G = 30, 2, 2
    for group_off in ([0, 25, 3, 40, -7, 30, 12, 2, 30],
                      [50, -1, 60, 29, 29, 0, 0, 31, 5],
                      [0, 30, 0, 30, 0, 30, 0, 30, 0]):
        for rank in (-1, 0, 1):
            _check(np.array(group_off), 8, E, G, rank, rows, 8)


@settings(max_examples=150, deadline=None)
@given(st.integers(1, 4), st.integers(1, 3), st.integers(1, 60), st.integers(-1, 3), st.data())
def test_random_offsets_stay_in_bounds(E, G, rows, rank, data):
    rank = rank if rank < G else -1
    num_groups = 2 * G * E
    group_off = data.draw(st.lists(st.integers(-10, rows + 10), min_size=num_groups + 1, max_size=num_groups + 1))
    gather = np.array(data.draw(st.lists(st.integers(-5, 3 * rows + 5), min_size=rows, max_size=rows)))
    _check(np.array(group_off), num_groups, E, G, rank, rows, data.draw(st.sampled_from([8, 64, 256])),
           gather=gather, gather_k=3, rows_x=rows)
