"""Helpers for the GPU parity tests: run one layer step through the C ABI on
seeded inputs and compare every stage with the CPU oracle.

The oracle is fed the GPU's own top-k indices for the integer stages (so a
near-tie decided differently in fp32 cannot cascade), and checks the gate
itself against its fp64 routing with the near-tie exclusion.
"""
from __future__ import annotations

import sys
import time
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np
import torch

from oracle import moe_oracle as O
from synth import workloads as W

NEAR_TIE = 1e-3
TOL = {"bf16": 2e-2, "f32": 1e-4}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


@dataclass
class LayerRun:
    cfg: W.MoEConfig
    li: W.LayerInputs
    w13: np.ndarray
    w2: np.ndarray
    shared: Optional[tuple]
    idx_pred: np.ndarray
    replica_cur: np.ndarray
    out: Dict[str, np.ndarray]
    x_perm_ok: Optional[bool]
    balancer: str = "libra"
    home_cur: Optional[np.ndarray] = None     # FreeBalance: placement of this step
    fb: Optional[tuple] = None                # FreeBalance: (tau, gamma num, gamma den, budget)


def run_layer(cfg: W.MoEConfig, layer: int = 1, step: int = 0, gather_rows: bool = True,
              materialize_x: bool = True, hs=None, weights=None, two_stage: bool = False,
              balancer: str = "libra", packed_weights: bool = False, overlap_split=None) -> LayerRun:
    from routed_expert_ffn_gate_amd.layer import MoELayer, to_device, to_host
    dev = torch.device("cuda")
    li = W.layer_inputs(cfg, layer, step, hs=hs)
    w13, w2 = weights if weights is not None else W.expert_weights_stacked(cfg, layer)
    sh = W.shared_weights(cfg)
    d = lambda a: to_device(a, cfg.dtype, dev)  # noqa: E731
    h, h_prev = d(li.h), d(li.h_prev)
    wc, wn = d(li.w_cur), d(li.w_next)
    bc, bn = d(li.b_cur), d(li.b_next)
    home = d(li.home)
    W13, W2 = d(w13), d(w2)
    S13 = S2 = None
    if sh is not None:
        S13, S2 = d(sh[0]), d(sh[1])
    if packed_weights:
        from routed_expert_ffn_gate_amd.layer import pack_expert_weights as pack
        W13, W2 = pack(W13), pack(W2)
        if sh is not None:
            S13, S2 = pack(S13), pack(S2)
    L = MoELayer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.inter, cfg.G, cfg.N, cfg.L, cfg.dtype, shared_inter=cfg.shared_inter,
                 gather_rows=gather_rows, materialize_x=materialize_x, balancer=balancer,
                 packed_weights=packed_weights, overlap_split=overlap_split)
    home_cur = None
    if balancer == "freebalance":
        replica_cur = torch.empty((cfg.G, 0), dtype=torch.int32, device=dev)
        home_cur = torch.empty((cfg.E,), dtype=torch.int32, device=dev)
        L.predict_placement(h_prev, wc, bc, home, home_cur)
        home_step = home_cur
    else:
        replica_cur = torch.empty((cfg.G, cfg.N), dtype=torch.int32, device=dev)
        L.predict_plan(h_prev, wc, bc, home, replica_cur)
        home_step = home
    idx_pred = L.idx_next.clone()
    run_step = L.step_two_stage if two_stage else L.step
    o = run_step(h, wc, bc, wn, bn, home_step, replica_cur, W13, W2, S13, S2)
    torch.cuda.synchronize()
    x_ok = None
    if o.x_perm is not None and materialize_x:
        from routed_expert_ffn_gate_amd import moelb as M
        # the row-copying permutation, on the same inputs, checked bit for bit
        M.moelb_permute(h, o.idx, cfg.G, home_step, replica_cur, o.host_count, L.ws_perm, o.group_off, o.perm,
                        o.pos, o.x_perm)
        torch.cuda.synchronize()
        src = h[(o.perm.long() // cfg.k)]
        x_ok = bool(torch.equal(o.x_perm.view(torch.int16) if cfg.dtype == "bf16" else o.x_perm.view(torch.int32),
                                src.view(torch.int16) if cfg.dtype == "bf16" else src.view(torch.int32)))
        del src
    out = {name: to_host(getattr(o, name)) for name in
           ["idx", "wts", "gap", "idx_next", "counts", "counts_next", "replica_next", "plan_load_next",
            "host_count", "load", "group_off", "perm", "pos", "y", "out"]}
    if o.shared is not None:
        out["shared"] = to_host(o.shared)
    fb = None
    if balancer == "freebalance":
        out["home_next"] = to_host(o.home_next)
        fb = (L.fb_tau, L.fb_gamma[0], L.fb_gamma[1], L.fb_budget)
    run = LayerRun(cfg, li, w13, w2, sh, to_host(idx_pred), to_host(replica_cur), out, x_ok, balancer,
                   to_host(home_cur) if home_cur is not None else None, fb)
    del L, W13, W2, h, h_prev
    torch.cuda.empty_cache()
    return run


def check_gate(run: LayerRun) -> dict:
    cfg, li, g = run.cfg, run.li, run.out
    idx_o, w_o, gap_o, idxn_o, z = O.route(li.h, li.w_cur, li.b_cur, li.w_next, li.b_next, cfg.k, cfg.dtype)
    h64 = O.widen(li.h, cfg.dtype)
    zn = O.router_logits(h64, O.widen(li.w_next, cfg.dtype), li.b_next)
    _, gapn_o = O.topk(zn, cfg.k)
    near = gap_o < NEAR_TIE
    near_n = gapn_o < NEAR_TIE
    T = cfg.T
    bad = 0
    worst_w = 0.0
    for t in range(T):
        if near[t]:
            continue
        so, sg = set(idx_o[t].tolist()), set(g["idx"][t].tolist())
        if so != sg:
            bad += 1
            continue
        wo = dict(zip(idx_o[t].tolist(), w_o[t].tolist()))
        for e, wg in zip(g["idx"][t].tolist(), g["wts"][t].tolist()):
            worst_w = max(worst_w, abs(wg - wo[e]) / wo[e])
    # exact order where the selected logits are well separated
    zs = -np.sort(-z, axis=1)[:, :cfg.k + 1]
    sep = np.all(np.diff(-zs, axis=1) >= NEAR_TIE, axis=1) if cfg.k < cfg.E else np.ones(T, bool)
    order_bad = int(np.sum(np.any(idx_o[sep] != g["idx"][sep], axis=1)))
    bad_next = 0
    for t in range(T):
        if near_n[t]:
            continue
        if set(idxn_o[t].tolist()) != set(g["idx_next"][t].tolist()):
            bad_next += 1
    gap_err = float(np.max(np.abs(g["gap"][~near] - gap_o[~near]))) if np.any(~near) else 0.0
    res = dict(near_ties=int(near.sum()), near_ties_next=int(near_n.sum()), idx_mismatch=bad,
               order_mismatch=order_bad, idx_next_mismatch=bad_next, max_rel_w=worst_w, max_gap_err=gap_err)
    assert bad == 0 and bad_next == 0 and order_bad == 0, res
    # router weights and the gap are fp32 outputs (fp32 logits from fp32
    # accumulation): the fp32 bar, relative for the weights, and in logit
    # units for the gap (a difference of two O(1..10) logits)
    assert worst_w <= TOL["f32"], res
    assert gap_err <= 1e-4, res
    return res


def check_integer_stages(run: LayerRun) -> dict:
    cfg, li, g = run.cfg, run.li, run.out
    G, E = cfg.G, cfg.E
    c = O.histogram(g["idx"], G, E)
    assert np.array_equal(g["counts"], c), "histogram (current)"
    cn = O.histogram(g["idx_next"], G, E)
    assert np.array_equal(g["counts_next"], cn), "histogram (lookahead)"
    cp = O.histogram(run.idx_pred, G, E)
    N = cfg.N
    home = li.home
    if run.balancer == "freebalance":
        from fractions import Fraction
        from oracle import swap_planner as SP
        tau, num, den, budget = run.fb
        home_cur, _, _ = SP.plan_swaps(cp, li.home, G, E, tau=tau, gamma=Fraction(num, den), max_swaps_per_rank=budget)
        assert np.array_equal(run.home_cur, home_cur), "swap plan (prologue)"
        home_next, _, pl = SP.plan_swaps(cn, li.home, G, E, tau=tau, gamma=Fraction(num, den),
                                         max_swaps_per_rank=budget)
        assert np.array_equal(g["home_next"], home_next), "swap plan (next layer)"
        assert np.array_equal(g["plan_load_next"], pl), "swap plan loads"
        home, N = home_cur, 0
        rep_cur = None
    elif N > 0:
        rep_cur = O.plan(cp, li.home, G, E, N, cfg.L)
        assert np.array_equal(run.replica_cur[:, :N], rep_cur), ("plan (prologue)", run.replica_cur, rep_cur)
        rep_next, pl = O.plan(cn, li.home, G, E, N, cfg.L, return_loads=True)
        assert np.array_equal(g["replica_next"][:, :N], rep_next), "plan (next layer)"
        assert np.array_equal(g["plan_load_next"], np.array(pl)), "plan loads"
    else:
        rep_cur = np.full((G, 1), -1, dtype=np.int32)
    hc, load = O.split(c, home, rep_cur if N > 0 else None, G, E, passes=12)
    assert np.array_equal(g["host_count"], hc), "split host_count"
    assert np.array_equal(g["load"], load), "split load"
    off, perm, pos = O.permute(g["idx"], home, rep_cur if N > 0 else None, hc, G, E)
    assert np.array_equal(g["group_off"], off), "permute group_off"
    assert np.array_equal(g["perm"][:len(perm)], perm), "permute perm"
    assert np.array_equal(g["pos"], pos), "permute pos"
    if run.x_perm_ok is not None:
        assert run.x_perm_ok, "x_perm rows are not bit copies of h rows"
    static = O.static_loads(c, li.home, G, E)
    return dict(spatial_static=O.spatial(static), spatial_split=O.spatial(load),
                lookahead_hit=O.lookahead_hit(run.idx_pred, g["idx"]))


def _row_rel(y, ref):
    den = np.max(np.abs(ref), axis=1)
    den = np.where(den == 0, 1.0, den)
    return np.max(np.abs(y - ref), axis=1) / den


def check_float_stages(run: LayerRun, tokens: Optional[np.ndarray] = None, seed: int = 0) -> dict:
    """Y rows of the sampled tokens' pairs and their combined outputs, against
    fp64 SwiGLU experts (GPU indices and weights), plus the dense MoE
    definition with the oracle's own routing on well-separated tokens.  One
    expert's weights are widened at a time."""
    cfg, li, g = run.cfg, run.li, run.out
    tol = TOL[cfg.dtype]
    T, k = cfg.T, cfg.k
    if tokens is None:
        tokens = np.arange(T)
    tokens = np.asarray(tokens)
    h64 = O.widen(li.h[tokens], cfg.dtype)
    idx_g, w_g, pos = g["idx"][tokens], g["wts"][tokens], g["pos"]
    idx_o, w_o, gap_o, _, _ = O.route(li.h[tokens], li.w_cur, li.b_cur, None, None, k, cfg.dtype)
    ref = np.zeros((len(tokens), cfg.d))
    dense = np.zeros((len(tokens), cfg.d))
    yerr = 0.0
    for e in np.unique(np.concatenate([idx_g.ravel(), idx_o.ravel()])):
        w13 = O.widen(run.w13[e], cfg.dtype)
        w2 = O.widen(run.w2[e], cfg.dtype)
        rg, cg = np.nonzero(idx_g == e)
        ro, co = np.nonzero(idx_o == e)
        rows = np.unique(np.concatenate([rg, ro]))
        y = O.swiglu(h64[rows], w13, w2)
        at = {int(r): i for i, r in enumerate(rows)}
        if len(rg):
            yr = y[[at[int(r)] for r in rg]]
            yq = O.widen(g["y"][pos[tokens[rg] * k + cg]], cfg.dtype)
            yerr = max(yerr, float(np.max(_row_rel(yq, yr))))
            ref[rg] += w_g[rg, cg][:, None] * yr
        if len(ro):
            dense[ro] += w_o[ro, co][:, None] * y[[at[int(r)] for r in ro]]
    serr = 0.0
    if run.shared is not None:
        s13, s2 = (O.widen(a, cfg.dtype) for a in run.shared)
        shared_ref = O.swiglu(h64, s13, s2)
        serr = float(np.max(_row_rel(O.widen(g["shared"][tokens], cfg.dtype), shared_ref)))
        ref += shared_ref
        dense += shared_ref
    out_g = O.widen(g["out"][tokens], cfg.dtype)
    oerr = float(np.max(_row_rel(out_g, ref)))
    keep = gap_o >= NEAR_TIE
    derr = float(np.max(_row_rel(out_g[keep], dense[keep]))) if np.any(keep) else 0.0
    res = dict(max_rel_y=yerr, max_rel_shared=serr, max_rel_out=oerr, max_rel_out_dense=derr, tokens=len(tokens))
    assert yerr <= tol and serr <= tol and oerr <= tol and derr <= tol, res
    return res


def sample_tokens(T: int, n: int, seed: int = 0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    pick = rng.choice(T, size=min(n, T), replace=False)
    return np.unique(np.concatenate([pick, [0, T - 1]])).astype(np.int64)
