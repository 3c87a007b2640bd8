"""GPU parity: every stage of the layer step, through the C ABI, against the
CPU oracle on identical seeded inputs.

Integer stages (histograms, plan, split, permutation) must be bit-exact when
fed the GPU's top-k indices; top-k must match except on near-ties (k-th minus
(k+1)-th logit < 1e-3); floats within 2e-2 (bf16) / 1e-4 (fp32) relative to an
fp64 oracle (per row, max-norm).
"""
import numpy as np
import pytest
import torch

from synth import workloads as W
from tests.gpu_layer import (check_float_stages, check_gate, check_integer_stages, log, run_layer,
                             sample_tokens)

pytestmark = pytest.mark.gpu


def _full_check(cfg, tokens=None, **kw):
    log(f"[layer] {cfg.name} T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} I={cfg.inter} G={cfg.G} N={cfg.N} "
        f"{cfg.dtype} {kw}")
    run = run_layer(cfg, **kw)
    r1 = check_gate(run)
    r2 = check_integer_stages(run)
    r3 = check_float_stages(run, tokens)
    log(f"  gate {r1}\n  int {r2}\n  float {r3}")
    return run


RAGGED = dict(T=200, d=200, E=24, k=3, inter=200, G=4, N=2, L=1)


def test_tiny_fp32_config(moelb):
    _full_check(W.config("c1_tiny_f32"))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_shapes(moelb, dtype):
    # tails everywhere: T not a multiple of the 128-token gate tile, d not a
    # multiple of the 64-wide K step, inter not a multiple of the 128-column
    # tile, E not a multiple of 32, odd k
    cfg = W.scaled(W.config("c2_qwen3_30b_decode"), dtype=dtype, steps=1, **RAGGED)
    _full_check(cfg)


def test_gather_equals_materialized(moelb):
    cfg = W.scaled(W.config("c2_qwen3_30b_decode"), steps=1, **RAGGED)
    a = run_layer(cfg, gather_rows=True, materialize_x=False)
    b = run_layer(cfg, gather_rows=False, materialize_x=True)
    assert b.x_perm_ok
    for key in ["y", "out", "perm", "pos", "group_off"]:
        assert np.array_equal(a.out[key], b.out[key]), key


def test_decode_steps_qwen3_30b_shape(moelb):
    cfg = W.config("c2_qwen3_30b_decode")
    weights = W.expert_weights_stacked(cfg, 1)
    for step in range(cfg.steps):
        log(f"[decode step {step}]")
        run = run_layer(cfg, step=step, weights=weights)
        check_gate(run)
        r = check_integer_stages(run)
        f = check_float_stages(run)
        log(f"  {r} {f}")


def test_prefill_qwen3_235b_shape(moelb):
    # every token: all 262144 Y rows and all 32768 output rows against fp64
    cfg = W.config("c3_qwen3_235b_prefill")
    _full_check(cfg)


def test_prefill_glm45_shape_with_shared_expert(moelb):
    cfg = W.config("c4_glm45_prefill")
    _full_check(cfg)


def test_drift_olmoe_shape_eight_layers(moelb):
    cfg = W.config("c5_olmoe_drift")
    hs = W.hidden_states(cfg, cfg.layers)
    for layer in range(1, cfg.layers + 1):
        log(f"[drift layer {layer}]")
        run = run_layer(cfg, layer=layer, hs=hs)
        check_gate(run)
        r = check_integer_stages(run)
        # every row on the first and the last layer (the two ends of the
        # drift), 512 sampled tokens on the layers between
        full = layer in (1, cfg.layers)
        f = check_float_stages(run, None if full else sample_tokens(cfg.T, 512, seed=layer))
        log(f"  {r} {f}")


@pytest.mark.parametrize("d,inter", [(576, 192), (320, 320), (192, 448), (128, 64)])
def test_persistent_gemms_short_k_several_tiles_per_workgroup(moelb, d, inter):
    # the persistent GEMMs at their shortest K (down: 3 and 5 steps of 64;
    # gate/up: 3 steps at d = 192), with more output tiles than workgroups and
    # column tails (gate/up: 448 = 3.5 x 128; down: 192 < 256); and below
    # three steps (2 and 1), the one-workgroup-per-tile direct-to-LDS kernels
    cfg = W.scaled(W.config("c2_qwen3_30b_decode"), steps=1, T=4096, d=d, E=32, k=8, inter=inter, G=8, N=2, L=1)
    _full_check(cfg, tokens=sample_tokens(cfg.T, 64))


@pytest.mark.parametrize("T,d,E,k,inter", [(512, 320, 64, 6, 192), (256, 64, 32, 4, 64), (1024, 2048, 128, 8, 768)])
def test_decode_tiles_64_rows(moelb, T, d, E, k, inter):
    # fewer than 128 rows per expert: the 64-row tile GEMMs, with column
    # tails (gate/up 192 = 1.5 x 128, down 320 = 1.25 x 256), one and three
    # 64-wide K steps, and a decode batch twice C2's
    cfg = W.scaled(W.config("c2_qwen3_30b_decode"), steps=1, T=T, d=d, E=E, k=k, inter=inter, G=8, N=2, L=1)
    assert T * k < 128 * E
    _full_check(cfg)


@pytest.mark.parametrize("name,changes", [
    ("c2_qwen3_30b_decode", dict(steps=1, **RAGGED)),
    ("c2_qwen3_30b_decode", dict(steps=1)),
    ("c4_glm45_prefill", dict(T=2048)),
])
def test_two_stage_step_identical_to_one_stage(moelb, name, changes):
    # MoE_local beside the split and remote permutation: the same step, bit
    # for bit, and the oracle's where checked
    cfg = W.scaled(W.config(name), **changes)
    a = run_layer(cfg)
    b = _full_check(cfg, tokens=sample_tokens(cfg.T, 32), two_stage=True)
    valid = a.out["pos"] >= 0
    for key in ["idx", "counts", "host_count", "load", "group_off", "perm", "pos", "replica_next", "out"]:
        assert np.array_equal(a.out[key], b.out[key]), key
    rows = a.out["pos"][valid]
    assert np.array_equal(a.out["y"][rows], b.out["y"][rows])


@pytest.mark.parametrize("name,changes", [
    ("c2_qwen3_30b_decode", dict(steps=1, **RAGGED)),
    ("c4_glm45_prefill", dict(T=2048)),
    ("c3_qwen3_235b_prefill", dict()),
])
def test_freebalance_layer_step(moelb, name, changes):
    # the same path with FreeBalance's swaps in place of replication: the
    # prologue and next-layer placements, the identity split, permutation,
    # FFN and combine against the oracle
    cfg = W.scaled(W.config(name), **changes)
    run = _full_check(cfg, tokens=sample_tokens(cfg.T, 24), balancer="freebalance")
    assert run.home_cur is not None
    assert np.array_equal(np.bincount(run.home_cur, minlength=cfg.G), np.bincount(run.li.home, minlength=cfg.G))


GRAPH_OUTPUTS = ("idx", "wts", "gap", "idx_next", "counts", "counts_next", "replica_next", "plan_load_next",
                 "host_count", "load", "group_off", "perm", "pos", "y", "out")


@pytest.mark.parametrize("name,changes,two_stage", [("c2_qwen3_30b_decode", {}, False),
                                                    ("c4_glm45_prefill", dict(T=2048), False),
                                                    ("c2_qwen3_30b_decode", RAGGED, False),
                                                    ("c4_glm45_prefill", dict(T=2048), True)])
def test_graph_replay_equals_eager(moelb, name, changes, two_stage):
    """The layer step captured once in a HIP graph (torch.cuda.CUDAGraph on the
    step's stream, the lookahead stream -- and for the two-stage step the
    split stream -- forked and joined by events) and replayed three times,
    each replay after an eager step on other inputs that overwrites every
    output: each replay reproduces the eager step's outputs bit for bit."""
    from routed_expert_ffn_gate_amd.layer import MoELayer, to_device
    cfg = W.scaled(W.config(name), **changes)
    log(f"[graph] {cfg.name} T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} shared={cfg.shared_inter} two_stage={two_stage}")
    dev = torch.device("cuda")
    up = lambda a: to_device(a, cfg.dtype, dev)  # noqa: E731
    li, li2 = W.layer_inputs(cfg, step=0), W.layer_inputs(cfg, step=1)
    w13, w2 = W.expert_weights_stacked(cfg, 1)
    sh = W.shared_weights(cfg)
    W13, W2 = up(w13), up(w2)
    S13, S2 = (up(sh[0]), up(sh[1])) if sh is not None else (None, None)
    args = [up(li.h), up(li.w_cur), up(li.b_cur), up(li.w_next), up(li.b_next), up(li.home)]
    args2 = [up(li2.h), up(li2.w_cur), up(li2.b_cur), up(li2.w_next), up(li2.b_next), up(li2.home)]
    L = MoELayer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.inter, cfg.G, cfg.N, cfg.L, cfg.dtype,
                 shared_inter=cfg.shared_inter, gather_rows=True, materialize_x=True)
    rep = torch.empty((cfg.G, cfg.N), dtype=torch.int32, device=dev)
    L.predict_plan(up(li.h_prev), args[1], args[2], args[5], rep)
    run = L.step_two_stage if two_stage else L.step
    step = lambda a: run(*a[:6], rep, W13, W2, S13, S2)  # noqa: E731
    o = step(args)
    torch.cuda.synchronize()
    ref = {n: getattr(o, n).clone() for n in GRAPH_OUTPUTS}
    if o.shared is not None:
        ref["shared"] = o.shared.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(args)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(args)
    torch.cuda.synchronize()
    for i in range(3):
        step(args2)
        torch.cuda.synchronize()
        assert not torch.equal(o.out, ref["out"])
        g.replay()
        torch.cuda.synchronize()
        for n, t in ref.items():
            assert torch.equal(getattr(o, n), t), (i, n)
    del g


def test_permute_two_phases_equal_one_call(moelb):
    from routed_expert_ffn_gate_amd import moelb as M
    dev = torch.device("cuda")
    rng = np.random.default_rng(21)
    for trial in range(12):
        G = int(rng.choice([1, 2, 4, 8]))
        E = G * int(rng.choice([1, 3, 8, 16]))
        k = int(rng.integers(1, 9))
        T = G * int(rng.choice([0, 1, 37, 200]))
        N = int(rng.integers(0, 4))
        d = 64
        pop = 1.0 / (1 + rng.permutation(E)) ** 1.2
        idx = rng.choice(E, size=(T, k), p=pop / pop.sum()).astype(np.int32)
        if T:
            idx[rng.random((T, k)) < 0.02] = -1  # pairs left out
        home = (np.arange(E) // (E // G)).astype(np.int32)
        rep = np.where(rng.random((G, max(N, 1))) < 0.8, rng.integers(0, E, (G, max(N, 1))), -1).astype(np.int32)
        t = lambda a: torch.from_numpy(a).to(dev)  # noqa: E731
        idx_t, home_t, rep_t = t(idx), t(home), t(rep)
        h = torch.randn((T, d), device=dev).to(torch.bfloat16)
        counts = torch.empty((G, E), dtype=torch.int32, device=dev)
        M.moelb_histogram(idx_t, G, counts)
        hc = torch.empty((E, G), dtype=torch.int32, device=dev)
        ld = torch.empty(G, dtype=torch.int32, device=dev)
        M.moelb_split(counts, home_t, rep_t if N else torch.full((G, 1), -1, dtype=torch.int32, device=dev), hc, ld,
                      passes=12)
        repn = rep_t[:, :N] if N else torch.empty((G, 0), dtype=torch.int32, device=dev)
        ws = torch.empty(M.moelb_permute_workspace_bytes(T, k, E, G), dtype=torch.uint8, device=dev)
        outs = []
        for two in (False, True):
            off = torch.full((2 * G * E + 1,), -9, dtype=torch.int32, device=dev)
            perm = torch.full((T * k,), -9, dtype=torch.int32, device=dev)
            pos = torch.full((T * k,), -9, dtype=torch.int32, device=dev)
            xp = torch.zeros((T * k, d), dtype=torch.bfloat16, device=dev)
            if two:
                M.moelb_permute_local(h, idx_t, G, home_t, repn, ws, off, perm, pos, xp)
                torch.cuda.synchronize()
                nl = int(off[G * E])
                ref = outs[0]
                assert torch.equal(off[:G * E + 1], ref[0][:G * E + 1]), trial
                assert torch.equal(perm[:nl], ref[1][:nl]), trial
                local = ref[2] < nl
                assert torch.equal(pos[local], ref[2][local]), trial
                assert bool((pos[~local] == -1).all()), trial
                M.moelb_permute_remote(h, idx_t, G, home_t, repn, hc, ws, off, perm, pos, xp)
            else:
                M.moelb_permute(h, idx_t, G, home_t, repn, hc, ws, off, perm, pos, xp)
            torch.cuda.synchronize()
            outs.append((off, perm, pos, xp.view(torch.int16)))
        for a, b in zip(*outs):
            assert torch.equal(a, b), trial


@pytest.mark.parametrize("T,k,E,G,N", [
    (512, 8, 128, 8, 2),     # decode shape, 4096 pairs
    (1024, 8, 256, 8, 8),    # 8192 pairs and E*G = 2048: the one-workgroup limits
    (1032, 8, 256, 8, 8),    # 8256 pairs: past the limit
    (128, 16, 32, 64, 8),    # 64 ranks, one segment each
    (96, 3, 48, 3, 1),       # 3 ranks cut into 6 pieces each, ragged pieces
    (2048, 4, 64, 16, 3),    # 16 ranks, one segment per wave
    (60, 16, 256, 4, 8),
    (7, 5, 13, 1, 0),        # one rank, no replicas
    (0, 4, 16, 4, 1),        # empty batch
])
def test_permute_one_workgroup_form(moelb, T, k, E, G, N):
    """moelb_permute without rows to copy runs batches of at most 8192 pairs
    with E*G <= 2048 in one workgroup; with rows it always takes the four-launch
    sort.  Both must give the oracle's outputs bit for bit: pairs left out,
    replica slots out of range, shares from the split and arbitrary shares
    (negative, short of or past the pool)."""
    from oracle import moe_oracle as O
    from routed_expert_ffn_gate_amd import moelb as M
    dev = torch.device("cuda")
    rng = np.random.default_rng(T * 131 + E * 7 + G)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)  # noqa: E731
    for trial in range(3):
        pop = 1.0 / (1 + rng.permutation(E)) ** 1.2
        idx = rng.choice(E, size=(T, k), p=pop / pop.sum()).astype(np.int32)
        if T:
            idx[rng.random((T, k)) < 0.02] = -1
            idx[rng.random((T, k)) < 0.01] = E + 3
        home = (np.arange(E) * G // E).astype(np.int32)
        rep = rng.integers(-2, E + 2, (G, max(N, 1))).astype(np.int32)[:, :N]
        idx_t, home_t, rep_t = t(idx), t(home), t(rep.reshape(G, N))
        if trial == 0:
            hc = rng.integers(-3, 40, (E, G)).astype(np.int32)
            hc_t = t(hc)
        else:
            counts = torch.empty((G, E), dtype=torch.int32, device=dev)
            M.moelb_histogram(idx_t, G, counts)
            hc_t = torch.empty((E, G), dtype=torch.int32, device=dev)
            ld = torch.empty(G, dtype=torch.int32, device=dev)
            rep_s = rep_t if N else torch.full((G, 1), -1, dtype=torch.int32, device=dev)
            M.moelb_split(counts, home_t, rep_s, hc_t, ld, passes=12 * (trial - 1))
            torch.cuda.synchronize()
            hc = hc_t.cpu().numpy()
        ws = torch.empty(M.moelb_permute_workspace_bytes(T, k, E, G), dtype=torch.uint8, device=dev)
        d = 64
        h = torch.randn((T, d), device=dev).to(torch.bfloat16)
        outs = []
        for rows in (False, True):
            off = torch.full((2 * G * E + 1,), -9, dtype=torch.int32, device=dev)
            perm = torch.full((T * k,), -9, dtype=torch.int32, device=dev)
            pos = torch.full((T * k,), -9, dtype=torch.int32, device=dev)
            xp = torch.zeros((T * k, d), dtype=torch.bfloat16, device=dev) if rows else None
            M.moelb_permute(h if rows else None, idx_t, G, home_t, rep_t, hc_t, ws, off, perm, pos, xp,
                            d=d, dtype=M.MOELB_BF16)
            torch.cuda.synchronize()
            outs.append([off.cpu().numpy(), perm.cpu().numpy(), pos.cpu().numpy()])
        ref = O.permute(idx, home, rep if N else None, hc, G, E)
        nvalid = int(ref[0][-1])
        for got in outs:
            np.testing.assert_array_equal(got[0], ref[0], err_msg=f"group_off trial {trial}")
            np.testing.assert_array_equal(got[1][:nvalid], ref[1], err_msg=f"perm trial {trial}")
            np.testing.assert_array_equal(got[2], ref[2], err_msg=f"pos trial {trial}")


def test_zero_router_single_hot_set(moelb):
    # W = 0: every token picks the same k experts (by bias), so a few groups
    # hold every pair -- the most skewed case the method has.
    cfg = W.scaled(W.config("c2_qwen3_30b_decode"), steps=1, T=256, d=256, inter=256)
    import synth.workloads as SW
    orig = SW.gate_params

    def zero_gate(c, gate_layer, step=0):
        w, b = orig(c, gate_layer, step)
        return np.zeros_like(w), b

    SW.gate_params = zero_gate
    try:
        run = run_layer(cfg)
    finally:
        SW.gate_params = orig
    check_gate(run)
    check_integer_stages(run)
    check_float_stages(run, sample_tokens(cfg.T, 32))
    assert len(np.unique(run.out["idx"])) == cfg.k


def test_limits_E256_k16_G64_N8(moelb):
    cfg = W.scaled(W.config("c2_qwen3_30b_decode"), steps=1, T=512, d=128, E=256, k=16, inter=64, G=64, N=8, L=4)
    _full_check(cfg)


def test_rank_share_covers_exactly_its_groups(moelb):
    from routed_expert_ffn_gate_amd import moelb as M
    from routed_expert_ffn_gate_amd.layer import MoELayer, to_device
    cfg = W.scaled(W.config("c2_qwen3_30b_decode"), steps=1, **RAGGED)
    run = run_layer(cfg, gather_rows=False, materialize_x=True)
    dev = torch.device("cuda")
    off = run.out["group_off"]
    G, E = cfg.G, cfg.E
    x = torch.from_numpy(np.ascontiguousarray(run.li.h).view(np.int16)).to(dev).view(torch.bfloat16)
    perm = torch.from_numpy(run.out["perm"]).to(dev)
    goff = torch.from_numpy(off).to(dev)
    w13 = to_device(run.w13, cfg.dtype, dev)
    w2 = to_device(run.w2, cfg.dtype, dev)
    P = cfg.T * cfg.k
    ws = torch.empty(M.moelb_grouped_ffn_workspace_bytes(P, 2 * G * E, E, cfg.d, cfg.inter, M.MOELB_BF16),
                     dtype=torch.uint8, device=dev)
    covered = np.zeros(P, dtype=bool)
    for r in range(G):
        y = torch.zeros((P, cfg.d), dtype=torch.bfloat16, device=dev)
        M.moelb_grouped_ffn(x, P, goff, E, w13, w2, ws, y, G=G, rank=r, gather=perm, gather_k=cfg.k)
        torch.cuda.synchronize()
        yh = y.view(torch.int16).cpu().numpy().view(np.uint16)
        mine = np.zeros(P, dtype=bool)
        for seg in range(2):
            for e in range(E):
                g = (seg * G + r) * E + e
                mine[off[g]:off[g + 1]] = True
        assert np.array_equal(yh[mine], run.out["y"][mine])
        assert not np.any(yh[~mine])
        covered |= mine
    assert covered.all()


def test_plan_and_split_random_instances(moelb):
    from oracle import moe_oracle as O
    from routed_expert_ffn_gate_amd import moelb as M
    dev = torch.device("cuda")
    rng = np.random.default_rng(11)
    for trial in range(120):
        G = int(rng.choice([2, 3, 4, 8, 16]))
        E = G * int(rng.choice([1, 2, 4, 8]))
        N = int(rng.integers(0, 5))
        L = int(rng.integers(0, N + 1))
        pop = 1.0 / (1 + rng.permutation(E)) ** rng.uniform(0.5, 1.6)
        c = np.stack([rng.multinomial(int(rng.integers(0, 400)), pop / pop.sum()) for _ in range(G)]).astype(np.int32)
        home = (np.arange(E) // (E // G)).astype(np.int32)
        ct = torch.from_numpy(c).to(dev)
        ht = torch.from_numpy(home).to(dev)
        rep = torch.full((G, max(N, 1)), -7, dtype=torch.int32, device=dev)
        pl = torch.empty(G, dtype=torch.int32, device=dev)
        if N > 0:
            M.moelb_plan(ct, ht, L, rep, pl)
            ref, loads = O.plan(c, home, G, E, N, L, return_loads=True)
            assert np.array_equal(rep.cpu().numpy(), ref), (trial, G, E, N, L)
            assert np.array_equal(pl.cpu().numpy(), loads)
            rep_in = ref
        else:
            rep_in = None
        passes = int(rng.choice([0, 1, 3, 12]))
        hc = torch.empty((E, G), dtype=torch.int32, device=dev)
        ld = torch.empty(G, dtype=torch.int32, device=dev)
        rt = torch.from_numpy(rep_in if rep_in is not None else np.full((G, 1), -1, np.int32)).to(dev)
        M.moelb_split(ct, ht, rt, hc, ld, passes=passes)
        hc_o, ld_o = O.split(c, home, rep_in, G, E, passes=passes)
        assert np.array_equal(hc.cpu().numpy(), hc_o), (trial, G, E, N, passes)
        assert np.array_equal(ld.cpu().numpy(), ld_o)


def test_split_variants_random_instances(moelb):
    """Each GPU split variant against its oracle, bit for bit, on random
    placements from the plan (register path up to 64 transfers, LDS path
    beyond)."""
    from oracle import moe_oracle as O
    from oracle import split_variants as V
    from routed_expert_ffn_gate_amd import moelb as M
    dev = torch.device("cuda")
    rng = np.random.default_rng(17)
    codes = {"relief": M.MOELB_SPLIT_RELIEF, "no_reverse": M.MOELB_SPLIT_NO_REVERSE,
             "jacobi": M.MOELB_SPLIT_JACOBI, "libra_greedy": M.MOELB_SPLIT_LIBRA_GREEDY,
             "water_fill": M.MOELB_SPLIT_WATER_FILL, "proportional": M.MOELB_SPLIT_PROPORTIONAL}
    for trial in range(48):
        G = int(rng.choice([2, 4, 8, 16, 64]))
        E = G * int(rng.choice([1, 2, 4])) if G < 64 else int(rng.choice([64, 128, 256]))
        N = int(rng.integers(1, 9 if G >= 16 else 4))
        L = int(rng.integers(0, N + 1))
        pop = 1.0 / (1 + rng.permutation(E)) ** rng.uniform(0.5, 1.6)
        c = np.stack([rng.multinomial(int(rng.integers(0, 3000)), pop / pop.sum()) for _ in range(G)]).astype(np.int32)
        home = (np.arange(E) // (E // G)).astype(np.int32)
        rep = O.plan(c[:, rng.permutation(E)] if trial % 2 else c, home, G, E, N, L)
        passes = int(rng.choice([0, 1, 3, 12]))
        ct, ht, rt = (torch.from_numpy(a).to(dev) for a in (c, home, rep))
        for name, code in codes.items():
            if name == "proportional" and G > 16:
                continue  # its exact arithmetic holds at most 16 hosts per expert
            eps = 0 if name in ("libra_greedy", "water_fill", "proportional") else int(rng.choice([0, 0, 2]))
            hc = torch.empty((E, G), dtype=torch.int32, device=dev)
            ld = torch.empty(G, dtype=torch.int32, device=dev)
            M.moelb_split_variant(ct, ht, rt, hc, ld, code, passes=passes, eps=eps)
            hc_o, ld_o = V.split_variant(c, home, rep, G, E, name, passes=passes, eps=eps)
            assert np.array_equal(hc.cpu().numpy(), hc_o), (trial, name, G, E, N, passes)
            assert np.array_equal(ld.cpu().numpy(), ld_o), (trial, name)


def test_split_proportional_large_loads(moelb):
    """The proportional split's exact shares (products of up to 15 host loads
    of about 2^26, several hundred bits) against the oracle's rationals, bit
    for bit, with 16 ranks whose experts have up to 16 hosts."""
    from oracle import moe_oracle as O
    from oracle import split_variants as V
    from routed_expert_ffn_gate_amd import moelb as M
    dev = torch.device("cuda")
    rng = np.random.default_rng(29)
    for trial in range(6):
        G, E, N = 16, int(rng.choice([16, 32])), 8
        L = int(rng.integers(0, N + 1))
        pop = 1.0 / (1 + rng.permutation(E)) ** rng.uniform(0.8, 1.4)
        c = np.stack([rng.multinomial(int(rng.integers(1 << 24, 1 << 26)), pop / pop.sum())
                      for _ in range(G)]).astype(np.int32)
        home = (np.arange(E) // (E // G)).astype(np.int32)
        rep = O.plan(c, home, G, E, N, L)
        hosts = 1 + np.array([(rep == e).any(axis=1).sum() for e in range(E)])
        log(f"[split proportional] trial {trial}: E={E} L={L} max hosts {hosts.max()}")
        ct, ht, rt = (torch.from_numpy(a).to(dev) for a in (c, home, rep))
        hc = torch.empty((E, G), dtype=torch.int32, device=dev)
        ld = torch.empty(G, dtype=torch.int32, device=dev)
        M.moelb_split_variant(ct, ht, rt, hc, ld, M.MOELB_SPLIT_PROPORTIONAL, passes=12)
        hc_o, ld_o = V.split_variant(c, home, rep, G, E, "proportional", passes=12)
        assert np.array_equal(hc.cpu().numpy(), hc_o), trial
        assert np.array_equal(ld.cpu().numpy(), ld_o), trial


def test_split_proportional_ties(moelb):
    """The proportional split where remainders tie or nearly tie, so that the
    ranking of the leftover tokens rests on exact remainders: equal counts on
    every rank (hosts with equal loads, equal remainders, ties to the lower
    rank), and counts near 2^22 that differ by 0-2 between cells (fractional
    shares within 1e-4 of each other whose exact remainders differ).  Bit for
    bit against the oracle's rationals."""
    from oracle import moe_oracle as O
    from oracle import split_variants as V
    from routed_expert_ffn_gate_amd import moelb as M
    dev = torch.device("cuda")
    rng = np.random.default_rng(31)
    cases = []
    for G, E, N, L, v in ((8, 16, 4, 2, 1000), (16, 32, 8, 4, 37), (4, 8, 3, 1, 5)):
        cases.append((G, E, N, L, np.full((G, E), v, dtype=np.int32)))
    for G, E, N, L in ((16, 16, 8, 4), (16, 32, 8, 8), (8, 16, 6, 3)):
        cases.append((G, E, N, L, ((1 << 22) + rng.integers(0, 3, size=(G, E))).astype(np.int32)))
    for i, (G, E, N, L, c) in enumerate(cases):
        home = (np.arange(E) // (E // G)).astype(np.int32)
        rep = O.plan(c, home, G, E, N, L)
        log(f"[split proportional ties] case {i}: G={G} E={E} N={N} L={L}")
        ct, ht, rt = (torch.from_numpy(a).to(dev) for a in (c, home, rep))
        hc = torch.empty((E, G), dtype=torch.int32, device=dev)
        ld = torch.empty(G, dtype=torch.int32, device=dev)
        M.moelb_split_variant(ct, ht, rt, hc, ld, M.MOELB_SPLIT_PROPORTIONAL, passes=12)
        hc_o, ld_o = V.split_variant(c, home, rep, G, E, "proportional", passes=12)
        assert np.array_equal(hc.cpu().numpy(), hc_o), i
        assert np.array_equal(ld.cpu().numpy(), ld_o), i

def test_split_stale_random_instances(moelb):
    """The stale split (an earlier step's shares dealt on new counts) against
    its oracle, bit for bit: earlier shares from the split of other counts on
    the same placement, from another placement, or random with zero and
    negative entries."""
    from oracle import moe_oracle as O
    from oracle import split_variants as V
    from routed_expert_ffn_gate_amd import moelb as M
    dev = torch.device("cuda")
    rng = np.random.default_rng(41)
    for trial in range(40):
        G = int(rng.choice([2, 4, 8, 16, 64]))
        E = G * int(rng.choice([1, 2, 4])) if G < 64 else int(rng.choice([64, 128, 256]))
        N = int(rng.integers(1, 9 if G >= 16 else 4))
        L = int(rng.integers(0, N + 1))
        pop = 1.0 / (1 + rng.permutation(E)) ** rng.uniform(0.5, 1.6)
        c0, c1 = (np.stack([rng.multinomial(int(rng.integers(0, 5000)), pop / pop.sum()) for _ in range(G)])
                  .astype(np.int32) for _ in range(2))
        home = (np.arange(E) // (E // G)).astype(np.int32)
        rep = O.plan(c0, home, G, E, N, L)
        kind = trial % 3
        if kind == 0:
            prev, _ = O.split(c0, home, rep, G, E)
        elif kind == 1:
            prev, _ = O.split(c0, home, O.plan(c1, home, G, E, N, L), G, E)
        else:
            prev = rng.integers(-3, 50, (E, G))
            prev[rng.random((E, G)) < 0.3] = 0
        prev = prev.astype(np.int32)
        ct, ht, rt, pt = (torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in (c1, home, rep, prev))
        hc = torch.empty((E, G), dtype=torch.int32, device=dev)
        ld = torch.empty(G, dtype=torch.int32, device=dev)
        M.moelb_split_stale(ct, ht, rt, pt, hc, ld)
        hc_o, ld_o = V.stale_split(c1, home, rep, prev, G, E)
        assert np.array_equal(hc.cpu().numpy(), hc_o), (trial, kind, G, E, N)
        assert np.array_equal(ld.cpu().numpy(), ld_o), (trial, kind)
        # the same step's shares reproduce the fresh split exactly
        if kind == 0:
            hcf = torch.empty_like(hc)
            M.moelb_split(torch.from_numpy(c0).to(dev), ht, rt, hcf, ld)
            M.moelb_split_stale(torch.from_numpy(c0).to(dev), ht, rt, hcf, hc, ld)
            assert torch.equal(hc, hcf), trial


def test_swap_planner_random_instances(moelb):
    """FreeBalance's swap planner against its oracle, bit for bit: placement,
    swap sequence and loads."""
    from fractions import Fraction
    from oracle import swap_planner as SP
    from routed_expert_ffn_gate_amd import moelb as M
    dev = torch.device("cuda")
    rng = np.random.default_rng(29)
    for trial in range(40):
        G = int(rng.choice([1, 2, 3, 8, 16, 64]))
        E = min(256, G * int(rng.choice([1, 2, 4, 8])))
        pop = 1.0 / (1 + rng.permutation(E)) ** rng.uniform(0.3, 1.6)
        c = np.stack([rng.multinomial(int(rng.integers(0, 20000)), pop / pop.sum()) for _ in range(G)]).astype(np.int32)
        home = rng.permutation(np.arange(E) // (E // G)).astype(np.int32)
        if trial % 5 == 0:
            home[rng.integers(0, E)] = -3  # read as rank 0
        num, den = int(rng.integers(0, 5)), int(rng.choice([1, 7, 1000, 1 << 20]))
        tau, budget = int(rng.choice([0, 0, 50])), int(rng.choice([0, 1, 2, 1 << 20]))
        ct, ht = torch.from_numpy(c).to(dev), torch.from_numpy(home).to(dev)
        ho = torch.empty(E, dtype=torch.int32, device=dev)
        ld = torch.empty(G, dtype=torch.int32, device=dev)
        sw = torch.full((E // 2 + 1, 2), -1, dtype=torch.int32, device=dev)
        ns = torch.empty(1, dtype=torch.int32, device=dev)
        M.moelb_plan_swaps(ct, ht, ho, ld, tau=tau, gamma=(num, den), max_swaps_per_rank=budget, swaps=sw, n_swaps=ns)
        where, swaps, load = SP.plan_swaps(c, home, G, E, tau=tau, gamma=Fraction(num, den),
                                           max_swaps_per_rank=budget)
        assert np.array_equal(ho.cpu().numpy(), where), trial
        assert np.array_equal(ld.cpu().numpy(), load), trial
        k = int(ns.item())
        assert k == len(swaps), trial
        assert [tuple(r) for r in sw.cpu().numpy()[:k].tolist()] == swaps, trial


def test_split_with_schedule_equals_without(moelb):
    """A schedule made for the placement gives the same split; one made for
    another placement (or garbage) is ignored and the split colours itself."""
    from oracle import moe_oracle as O
    from routed_expert_ffn_gate_amd import moelb as M
    dev = torch.device("cuda")
    rng = np.random.default_rng(23)
    for trial in range(20):
        G = int(rng.choice([2, 4, 8, 16, 64]))
        E = G * int(rng.choice([1, 2, 4])) if G < 64 else 256
        N = int(rng.integers(1, 9 if G >= 16 else 4))
        pop = 1.0 / (1 + rng.permutation(E)) ** 1.2
        c = np.stack([rng.multinomial(2000, pop / pop.sum()) for _ in range(G)]).astype(np.int32)
        home = (np.arange(E) // (E // G)).astype(np.int32)
        rep = O.plan(c, home, G, E, N, N // 2)
        rep2 = O.plan(c[:, ::-1].copy(), home, G, E, N, N // 2)
        ct, ht, rt, rt2 = (torch.from_numpy(a).to(dev) for a in (c, home, rep, rep2))
        ref_hc = torch.empty((E, G), dtype=torch.int32, device=dev)
        ref_ld = torch.empty(G, dtype=torch.int32, device=dev)
        M.moelb_split(ct, ht, rt, ref_hc, ref_ld, passes=12)
        sched = torch.full((M.MOELB_SPLIT_SCHEDULE_INTS,), -1, dtype=torch.int32, device=dev)
        other = torch.full_like(sched, -1)
        M.moelb_split_schedule(ht, rt, sched, G)
        M.moelb_split_schedule(ht, rt2, other, G)
        garbage = torch.from_numpy(rng.integers(-5, 40, M.MOELB_SPLIT_SCHEDULE_INTS).astype(np.int32)).to(dev)
        for sc in (sched, other, garbage, None):
            hc = torch.empty_like(ref_hc)
            ld = torch.empty_like(ref_ld)
            M.moelb_split_scheduled(ct, ht, rt, sc, hc, ld, passes=12)
            assert torch.equal(hc, ref_hc) and torch.equal(ld, ref_ld), trial
        # the schedule itself: n transfers, each colour class rank-disjoint
        sh = sched.cpu().numpy()
        n, ncol = int(sh[0]), int(sh[1])
        tr = sh[2:2 + 3 * n].reshape(n, 3) if n else np.zeros((0, 3), np.int32)
        transfers = O.split_transfers(home, O.host_sets(home, rep, E), E)
        assert n == len(transfers)
        assert [(int(u), int(v)) for u, v, _ in tr] == [(u, v) for u, v, _ in transfers]
        assert tr[:, 2].tolist() == O.colour_transfers(transfers)
        for col in range(ncol):
            ranks = tr[tr[:, 2] == col][:, :2].ravel()
            assert len(ranks) == len(set(ranks.tolist())), (trial, col)


def test_split_heavily_replicated_home(moelb):
    """Every rank replicates the four experts of rank 0: rank 0 ends up in one
    transfer per replica, which takes the split past 64 edge colours (and, at
    G=16, just below)."""
    from oracle import moe_oracle as O
    from routed_expert_ffn_gate_amd import moelb as M
    dev = torch.device("cuda")
    rng = np.random.default_rng(5)
    for G in (16, 32, 64):
        E, N = 4 * G, 8
        home = (np.arange(E) // 4).astype(np.int32)
        rep = np.empty((G, N), np.int32)
        for r in range(G):
            if r == 0:
                rep[r] = [4 + j for j in range(4)] + [8 + j for j in range(4)]
            else:
                nxt = (r + 1) % G or 1  # a rank other than r and 0
                rep[r] = [0, 1, 2, 3] + [4 * nxt + j for j in range(4)]
        pop = np.ones(E)
        pop[:4] = 40.0
        c = np.stack([rng.multinomial(4000, pop / pop.sum()) for _ in range(G)]).astype(np.int32)
        hc = torch.empty((E, G), dtype=torch.int32, device=dev)
        ld = torch.empty(G, dtype=torch.int32, device=dev)
        M.moelb_split(torch.from_numpy(c).to(dev), torch.from_numpy(home).to(dev), torch.from_numpy(rep).to(dev),
                      hc, ld, passes=12)
        hc_o, ld_o = O.split(c, home, rep, G, E, passes=12)
        assert np.array_equal(hc.cpu().numpy(), hc_o), G
        assert np.array_equal(ld.cpu().numpy(), ld_o), G


def test_empty_batch(moelb):
    from routed_expert_ffn_gate_amd import moelb as M
    dev = torch.device("cuda")
    E, k, d, G = 8, 2, 64, 4
    h = torch.empty((0, d), dtype=torch.bfloat16, device=dev)
    w = torch.zeros((E, d), dtype=torch.bfloat16, device=dev)
    b = torch.zeros(E, dtype=torch.float32, device=dev)
    idx = torch.empty((0, k), dtype=torch.int32, device=dev)
    wts = torch.empty((0, k), dtype=torch.float32, device=dev)
    M.moelb_gate_topk(h, w, b, None, None, idx, wts)
    counts = torch.full((G, E), 5, dtype=torch.int32, device=dev)
    M.moelb_histogram(idx, G, counts)
    torch.cuda.synchronize()
    assert int(counts.abs().sum()) == 0
    out = torch.empty((0, d), dtype=torch.bfloat16, device=dev)
    y = torch.empty((0, d), dtype=torch.bfloat16, device=dev)
    pos = torch.empty((0,), dtype=torch.int32, device=dev)
    M.moelb_combine(y, pos, wts, out)
    torch.cuda.synchronize()


def _fast_bucket(z32):
    """Top 24 bits of the order-preserving bit pattern of fp32 logits: the
    bucket a 32-bit selection key with an 8-bit id would keep."""
    b = z32.astype(np.float32).view(np.uint32).astype(np.uint64)
    ordered = np.where(b & 0x80000000, b ^ 0xFFFFFFFF, b ^ 0x80000000)
    return ordered >> 8


@pytest.mark.parametrize("E,k", [(32, 4), (64, 8)])
def test_topk_exact_at_large_logits(moelb, E, k):
    # Logits near +100 (current router) and -100 (lookahead) on a grid of
    # 2^-11: the fp32 logits are exact, neighbours 3 grid steps apart (1.5e-3,
    # outside the 1e-3 near-tie band) can share a 2^-9-wide bucket of a 24-bit
    # key, so ranking by truncated keys would misorder or mis-select them.
    from routed_expert_ffn_gate_amd import moelb as M
    from routed_expert_ffn_gate_amd.layer import to_device, to_host
    from oracle import moe_oracle as O
    T, d = 1024, 128
    rng = np.random.default_rng(11)
    h = np.zeros((T, d), np.float32)
    h[np.arange(T), np.arange(T) % 64] = 1.0
    wc = np.zeros((E, d), np.float32)
    wn = np.zeros((E, d), np.float32)
    wc[:, :64] = rng.integers(0, 128, size=(E, 64)) * 2.0 ** -11
    wn[:, :64] = rng.integers(0, 128, size=(E, 64)) * 2.0 ** -11
    bf = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)  # exact: every value fits bf16  # noqa: E731
    h16, wc16, wn16 = bf(h), bf(wc), bf(wn)
    bc = np.full(E, 100.0, np.float32)
    bn = np.full(E, -100.0, np.float32)
    idx_o, w_o, gap_o, idxn_o, z = O.route(h16, wc16, bc, wn16, bn, k, "bf16")
    zn = O.router_logits(O.widen(h16, "bf16"), O.widen(wn16, "bf16"), bn)
    _, gapn_o = O.topk(zn, k)
    # the workload must contain tokens that ranking by a 24-bit key (ties by
    # id) would decide wrongly outside the near-tie band
    hard = 0
    for zz, gg, io in ((z, gap_o, idx_o), (zn, gapn_o, idxn_o)):
        key = (_fast_bucket(zz) << np.uint64(8)) | (255 - np.arange(E)).astype(np.uint64)[None, :]
        sel = np.argsort(-key.astype(np.float64), axis=1, kind="stable")[:, :k]
        hard += int(np.sum(np.any(np.sort(sel, 1) != np.sort(io, 1), axis=1) & (gg >= 1e-3)))
    assert hard > 0
    dev = torch.device("cuda")
    up = lambda a: to_device(a, "bf16", dev)  # noqa: E731
    i32 = dict(dtype=torch.int32, device=dev)
    idx, idx_next = torch.empty((T, k), **i32), torch.empty((T, k), **i32)
    wts = torch.empty((T, k), dtype=torch.float32, device=dev)
    gap = torch.empty((T,), dtype=torch.float32, device=dev)
    M.moelb_gate_topk(up(h16), up(wc16), torch.from_numpy(bc).to(dev), up(wn16), torch.from_numpy(bn).to(dev),
                      idx, wts, gap, idx_next)
    torch.cuda.synchronize()
    gi, gw, gg, gn = to_host(idx), to_host(wts), to_host(gap), to_host(idx_next)
    keep, keep_n = gap_o >= 1e-3, gapn_o >= 1e-3
    log(f"[topk large logits] E={E} k={k}: {hard} tokens a 24-bit key would mis-select, "
        f"{int((~keep).sum())}/{int((~keep_n).sum())} near-ties excluded")
    # sets exact outside near-ties; order exact where the top k+1 are separated
    assert np.array_equal(np.sort(gi[keep], 1), np.sort(idx_o[keep], 1))
    assert np.array_equal(np.sort(gn[keep_n], 1), np.sort(idxn_o[keep_n], 1))
    zs = -np.sort(-z, axis=1)[:, :k + 1]
    sep = np.all(-np.diff(zs, axis=1) >= 1e-3, axis=1)
    assert np.array_equal(gi[sep], idx_o[sep])
    assert np.max(np.abs(gg[keep] - gap_o[keep])) <= 1e-4
    assert np.max(np.abs(gw[keep] - w_o[keep]) / w_o[keep]) <= 1e-4


def test_pack_weights_layout(moelb):
    """moelb_pack_weights against the layout written out with numpy:
    [E][rows][K] -> [E][rows/8][K/64][8][64], bit for bit."""
    from routed_expert_ffn_gate_amd import moelb as M
    dev = torch.device("cuda")
    rng = np.random.default_rng(3)
    for E, rows, K in [(3, 16, 64), (2, 24, 192), (5, 1536, 2048)]:
        w = rng.integers(-32768, 32768, (E, rows, K), dtype=np.int64).astype(np.int16)
        wt = torch.from_numpy(w).to(dev).view(torch.bfloat16)
        out = torch.empty_like(wt)
        M.moelb_pack_weights(wt, out)
        torch.cuda.synchronize()
        ref = w.reshape(E, rows // 8, 8, K // 64, 64).transpose(0, 1, 3, 2, 4).reshape(E, rows, K)
        assert np.array_equal(out.view(torch.int16).cpu().numpy(), ref), (E, rows, K)


@pytest.mark.parametrize("changes", [
    dict(T=256, d=512, E=32, k=4, inter=256, G=4, N=2, L=1),    # 64-row decode tiles
    dict(T=2048, d=512, E=8, k=2, inter=256, G=4, N=2, L=1),    # persistent GEMMs
    dict(T=1024, d=128, E=8, k=2, inter=128, G=4, N=2, L=1),    # K/64 = 2: one workgroup per tile
])
def test_packed_weights_equal_row_major(moelb, changes):
    """The layer step with weights packed by moelb_pack_weights: every output
    equal to the row-major step's, bit for bit, and the oracle's."""
    cfg = W.scaled(W.config("c2_qwen3_30b_decode"), steps=1, **changes)
    a = run_layer(cfg)
    b = _full_check(cfg, tokens=sample_tokens(cfg.T, 32), packed_weights=True)
    for key in ["group_off", "perm", "pos", "y", "out"]:
        assert np.array_equal(a.out[key], b.out[key]), key


def test_packed_weights_shared_expert(moelb):
    cfg = W.scaled(W.config("c4_glm45_prefill"), T=1024)
    a = run_layer(cfg)
    b = run_layer(cfg, packed_weights=True)
    for key in ["y", "shared", "out"]:
        assert np.array_equal(a.out[key], b.out[key]), key


@pytest.mark.parametrize("T,d,E,k,dtype,look", [
    (300, 256, 8, 8, "bf16", True),      # k = E: every expert selected, gap +inf
    (300, 256, 64, 1, "bf16", True),     # k = 1
    (132, 200, 40, 4, "bf16", False),    # d % 64 != 0 (register-staged kernel), no lookahead router
    (260, 128, 256, 16, "bf16", True),   # E = 256, k = 16
    (100, 96, 16, 16, "f32", True),      # fp32, k = E
    (4096, 512, 128, 8, "bf16", False),  # 64-token blocks, current router only
    (16100, 128, 64, 8, "bf16", True),   # 128-token blocks, one launch per router, ragged last block
    (20000, 128, 32, 4, "bf16", True),   # 128-token blocks, both routers in one launch, ragged
    (20000, 128, 64, 4, "bf16", False),  # 128-token blocks, current router only, ragged
])
def test_gate_edge_shapes(moelb, T, d, E, k, dtype, look):
    """moelb_gate_topk alone against the oracle's route on the edges of its
    shape space: the selected set and, where the logits are separated, its
    order; weights to the fp32 bar; the gap (+inf when k = E); the lookahead
    indices."""
    from oracle import moe_oracle as O
    from routed_expert_ffn_gate_amd import moelb as M
    from routed_expert_ffn_gate_amd.layer import to_device
    from tests.gpu_layer import NEAR_TIE, TOL
    cfg = W.scaled(W.config("c2_qwen3_30b_decode"), steps=1, T=T, d=d, E=E, k=k, inter=64, G=4, N=1, L=1,
                   dtype=dtype)
    li = W.layer_inputs(cfg)
    dev = torch.device("cuda")
    up = lambda a: to_device(a, dtype, dev)  # noqa: E731
    h, wc, wn = up(li.h), up(li.w_cur), up(li.w_next)
    bc, bn = up(li.b_cur), up(li.b_next)
    idx = torch.full((T, k), -7, dtype=torch.int32, device=dev)
    wts = torch.zeros((T, k), dtype=torch.float32, device=dev)
    gap = torch.zeros(T, dtype=torch.float32, device=dev)
    idxn = torch.full((T, k), -7, dtype=torch.int32, device=dev) if look else None
    M.moelb_gate_topk(h, wc, bc, wn if look else None, bn if look else None, idx, wts, gap, idxn)
    torch.cuda.synchronize()
    idx_o, w_o, gap_o, idxn_o, z = O.route(li.h, li.w_cur, li.b_cur, li.w_next if look else None,
                                           li.b_next if look else None, k, dtype)
    g_idx, g_w, g_gap = idx.cpu().numpy(), wts.cpu().numpy(), gap.cpu().numpy()
    near = gap_o < NEAR_TIE
    assert np.all((g_idx >= 0) & (g_idx < E))
    zs = -np.sort(-z, axis=1)[:, :min(k + 1, E)]
    sep = np.all(np.diff(-zs, axis=1) >= NEAR_TIE, axis=1)
    for t in range(T):
        if near[t]:
            continue
        assert set(g_idx[t].tolist()) == set(idx_o[t].tolist()), t
        if sep[t]:
            assert g_idx[t].tolist() == idx_o[t].tolist(), t
        wo = dict(zip(idx_o[t].tolist(), w_o[t].tolist()))
        for e, wg in zip(g_idx[t].tolist(), g_w[t].tolist()):
            assert abs(wg - wo[e]) <= TOL["f32"] * wo[e], (t, e)
    if k == E:
        assert np.all(np.isinf(g_gap) & (g_gap > 0))
    else:
        assert np.max(np.abs(g_gap[~near] - gap_o[~near])) <= 1e-4
    if look:
        zn = O.router_logits(O.widen(li.h, dtype), O.widen(li.w_next, dtype), li.b_next)
        _, gapn = O.topk(zn, k)
        gn = idxn.cpu().numpy()
        for t in range(T):
            if gapn[t] >= NEAR_TIE:
                assert set(gn[t].tolist()) == set(idxn_o[t].tolist()), t


@pytest.mark.parametrize("T,k,d,rows_y,dtype,shared", [
    (64, 1, 8, 64, "bf16", False),
    (100, 3, 200, 250, "bf16", True),
    (257, 8, 4096, 1900, "bf16", False),
    (33, 16, 136, 500, "f32", True),
])
def test_combine_left_out_pairs(moelb, T, k, d, rows_y, dtype, shared):
    """moelb_combine against the oracle: positions < 0 or >= rows_y (pairs
    left out) contribute nothing; per-row max-norm error at the dtype's bar."""
    from oracle import moe_oracle as O
    from routed_expert_ffn_gate_amd import moelb as M
    from tests.gpu_layer import TOL, _row_rel
    dev = torch.device("cuda")
    rng = np.random.default_rng(T * 7 + k)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    y = torch.randn((rows_y, d), device=dev).to(tdt)
    pos = rng.integers(0, rows_y, T * k)
    drop = rng.random(T * k)
    pos[drop < 0.1] = -1
    pos[(drop >= 0.1) & (drop < 0.15)] = rows_y + rng.integers(0, 5, int(((drop >= 0.1) & (drop < 0.15)).sum()))
    wts = rng.random((T, k)).astype(np.float32)
    sh = torch.randn((T, d), device=dev).to(tdt) if shared else None
    out = torch.full((T, d), 3.0, device=dev).to(tdt)
    M.moelb_combine(y, torch.from_numpy(pos.astype(np.int32)).to(dev), torch.from_numpy(wts).to(dev), out,
                    shared=sh)
    torch.cuda.synchronize()
    widen = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    pos_o = np.where(pos < rows_y, pos, -1)
    ref = O.combine(widen(y), pos_o, wts, T, k, widen(sh) if shared else None)
    err = _row_rel(widen(out), ref)
    assert float(np.max(err)) <= TOL[dtype], float(np.max(err))


@pytest.mark.parametrize("T,k,E,G,hot", [
    (512, 8, 128, 8, 0.0),
    (4096, 2, 16, 4, 0.9),       # one expert takes 90 % of the pairs
    (64 * 100, 16, 256, 64, 0.3),
    (12, 1, 3, 3, 0.0),
])
def test_histogram_invalid_ids_and_hot_expert(moelb, T, k, E, G, hot):
    """moelb_histogram against the oracle, bit for bit: ids outside [0, E)
    skipped, a hot expert (the one-atomic-per-wave path), column sums."""
    from oracle import moe_oracle as O
    from routed_expert_ffn_gate_amd import moelb as M
    dev = torch.device("cuda")
    rng = np.random.default_rng(T + E)
    idx = rng.integers(0, E, (T, k))
    idx[rng.random((T, k)) < hot] = E // 2
    r = rng.random((T, k))
    idx[r < 0.03] = -1
    idx[(r >= 0.03) & (r < 0.05)] = E + 7
    idx = idx.astype(np.int32)
    counts = torch.full((G, E), -5, dtype=torch.int32, device=dev)
    total = torch.full((E,), -5, dtype=torch.int32, device=dev)
    M.moelb_histogram(torch.from_numpy(idx).to(dev), G, counts, expert_total=total)
    torch.cuda.synchronize()
    ref = O.histogram(idx, G, E)
    assert np.array_equal(counts.cpu().numpy(), ref)
    assert np.array_equal(total.cpu().numpy(), ref.sum(0))


@pytest.mark.parametrize("name,changes", [
    ("c2_qwen3_30b_decode", dict(steps=1, **RAGGED)),
    ("c4_glm45_prefill", dict(T=2048)),
    ("c2_qwen3_30b_decode", dict(steps=1, T=2048, d=256, inter=256, G=64, N=8, L=4, E=256, k=4)),
])
def test_split_beside_local_permutation(moelb, name, changes):
    """The step with the split on its own stream beside the local half of the
    permutation equals the step with both in sequence, bit for bit."""
    cfg = W.scaled(W.config(name), **changes)
    a = run_layer(cfg, overlap_split=False)
    b = run_layer(cfg, overlap_split=True)
    for key in ["host_count", "load", "group_off", "perm", "pos", "y", "out"]:
        assert np.array_equal(a.out[key], b.out[key]), key
