"""GPU: the grouped FFN's schedule tables equal their model (expert-major
virtual rows, M tiles, row map) on device offsets that increase, and on
offsets that decrease, overlap and leave [0, rows]; on the latter every row
the schedule computes holds one of its computing groups' results, the others
are untouched, and nothing outside y is written."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from tests import ffn_schedule_model as F
from tests.gpu_layer import TOL, _row_rel, log

pytestmark = pytest.mark.gpu

E, G, D, INTER, ROWS = 2, 2, 256, 192, 700
CASES = {
    "increasing": [0, 90, 90, 300, 301, 420, 500, 520, 700],
    "decreasing_overlapping_out_of_range": [0, 400, 120, 650, -30, 260, 800, 300, 90],
}


def _setup(group_off):
    from routed_expert_ffn_gate_amd import moelb as M
    dev = torch.device("cuda")
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((ROWS, D)) * 1.0).astype(np.float32)
    w13 = (rng.standard_normal((E, 2 * INTER, D)) * 0.05).astype(np.float32)
    w2 = (rng.standard_normal((E, D, INTER)) * 0.05).astype(np.float32)
    bf = lambda a: torch.from_numpy(a).to(dev).to(torch.bfloat16)  # noqa: E731
    X, W13, W2 = bf(x), bf(w13), bf(w2)
    off = torch.tensor(group_off, dtype=torch.int32, device=dev)
    nbytes = M.moelb_grouped_ffn_workspace_bytes(ROWS, len(group_off) - 1, E, D, INTER, M.MOELB_BF16)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    return M, X, W13, W2, off, ws


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("rank", [-1, 1])
def test_schedule_tables_equal_model(moelb, case, rank):
    group_off = CASES[case]
    ng = len(group_off) - 1
    log(f"[ffn schedule] {case} rank={rank}")
    M, X, W13, W2, off, ws = _setup(group_off)
    ws.fill_(0xAB)  # tables are written, not assumed zero
    y = torch.zeros((ROWS, D), dtype=torch.bfloat16, device=X.device)
    M.moelb_grouped_ffn_stages(M.MOELB_FFN_SCHEDULE, X, ROWS, off, E, W13, W2, ws, y, G=G, rank=rank)
    torch.cuda.synchronize()
    eoff, gvb, tiles = F.schedule(np.array(group_off), ng, E, G, rank, ROWS, 256)
    rm, src = F.rowmap(np.array(group_off), ng, E, ROWS, eoff, gvb)
    o = F.workspace_offsets(ROWS, ng, E, INTER, 2)
    w = ws.cpu().numpy()
    i32 = lambda name, n: w[o[name]:o[name] + 4 * n].view(np.int32)  # noqa: E731
    assert i32("eoff", E + 1).tolist() == eoff
    assert i32("gvb", ng).tolist() == gvb
    nt = int(i32("n_mtiles", 1)[0])
    assert nt == len(tiles)
    assert list(zip(i32("mt_e", nt).tolist(), i32("mt_v0", nt).tolist())) == tiles
    assert np.array_equal(i32("rowmap", eoff[E]), rm)
    assert np.array_equal(i32("asrc", eoff[E]), src)


@pytest.mark.parametrize("case", list(CASES))
def test_ffn_rows_on_any_offsets(moelb, case):
    group_off = CASES[case]
    ng = len(group_off) - 1
    log(f"[ffn rows] {case}")
    M, X, W13, W2, off, ws = _setup(group_off)
    sentinel = torch.full((ROWS + 64, D), 7.0, dtype=torch.bfloat16, device=X.device)
    y = sentinel[:ROWS]
    M.moelb_grouped_ffn(X, ROWS, off, E, W13, W2, ws, y, G=G)
    torch.cuda.synchronize()
    widen = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    x64, w13, w2 = widen(X), widen(W13), widen(W2)
    ref = [O.swiglu(x64, w13[e], w2[e]) for e in range(E)]
    yg = widen(y)
    assert np.all(widen(sentinel[ROWS:]) == 7.0)  # nothing written past y
    # the rows the schedule computes, and with which expert: virtual row v <
    # eoff[E] of expert e computes physical row rowmap[v]
    eoff, gvb, _ = F.schedule(np.array(group_off), ng, E, G, -1, ROWS, 256)
    rm, _ = F.rowmap(np.array(group_off), ng, E, ROWS, eoff, gvb)
    computed = [set() for _ in range(ROWS)]
    for e in range(E):
        for v in range(eoff[e], eoff[e + 1]):
            computed[rm[v]].add(e)
    worst = 0.0
    for q in range(ROWS):
        if not computed[q]:
            assert np.all(yg[q] == 7.0), q  # rows no group computes are not written
            continue
        errs = [float(_row_rel(yg[q:q + 1], ref[e][q:q + 1])[0]) for e in sorted(computed[q])]
        worst = max(worst, min(errs))
    log(f"  max rel err {worst:.3g}")
    assert worst <= TOL["bf16"]


@pytest.mark.parametrize("ng", [4096, 4100])
@pytest.mark.parametrize("rank", [-1, 3])
def test_schedule_tables_many_groups(moelb, ng, rank):
    """Up to 4096 groups the schedule and the row map run as one launch (each
    workgroup derives the tables from group_off in LDS); past that as two.
    Both give the model's tables, on offsets that mostly increase, with
    some that decrease or leave [0, rows]."""
    from routed_expert_ffn_gate_amd import moelb as M
    e_, g_, rows = 4, 8, 3000
    rng = np.random.default_rng(ng + rank)
    steps = rng.integers(0, 2, ng + 1)
    group_off = np.minimum(np.cumsum(steps) - steps[0], rows)
    bad = rng.random(ng + 1) < 0.02
    group_off[bad] += rng.integers(-40, 40, int(bad.sum()))  # local decreases and overlaps
    group_off[-1] = rows + 25  # past the rows
    group_off = group_off.astype(np.int32).tolist()
    log(f"[ffn schedule] {ng} groups rank={rank}")
    dev = torch.device("cuda")
    x = torch.zeros((rows, D), dtype=torch.bfloat16, device=dev)
    w13 = torch.zeros((e_, 2 * INTER, D), dtype=torch.bfloat16, device=dev)
    w2 = torch.zeros((e_, D, INTER), dtype=torch.bfloat16, device=dev)
    off = torch.tensor(group_off, dtype=torch.int32, device=dev)
    nbytes = M.moelb_grouped_ffn_workspace_bytes(rows, ng, e_, D, INTER, M.MOELB_BF16)
    ws = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device=dev)
    y = torch.zeros((rows, D), dtype=torch.bfloat16, device=dev)
    M.moelb_grouped_ffn_stages(M.MOELB_FFN_SCHEDULE, x, rows, off, e_, w13, w2, ws, y, G=g_, rank=rank)
    torch.cuda.synchronize()
    eoff, gvb, tiles = F.schedule(np.array(group_off), ng, e_, g_, rank, rows, 256)
    rm, src = F.rowmap(np.array(group_off), ng, e_, rows, eoff, gvb)
    o = F.workspace_offsets(rows, ng, e_, INTER, 2)
    w = ws.cpu().numpy()
    i32 = lambda name, n: w[o[name]:o[name] + 4 * n].view(np.int32)  # noqa: E731
    assert i32("eoff", e_ + 1).tolist() == eoff
    assert i32("gvb", ng).tolist() == gvb
    nt = int(i32("n_mtiles", 1)[0])
    assert nt == len(tiles)
    assert list(zip(i32("mt_e", nt).tolist(), i32("mt_v0", nt).tolist())) == tiles
    assert np.array_equal(i32("rowmap", eoff[e_]), rm)
    assert np.array_equal(i32("asrc", eoff[e_]), src)
