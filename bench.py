#!/usr/bin/env python3
"""MoE-layer throughput of the routing-and-balancing hot path on one MI355X.

One step = one whole layer step on one batch: gate + lookahead gate, two
histograms, plan for the next layer, Relief split, permutation, grouped
SwiGLU FFN (+ shared expert where the workload has one) and combine.  Inputs
are seeded synthetic tensors of the workload's shapes, resident in HBM before
the timed region.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload NAME]

Traffic counters: run under ``rocprofv3 --pmc FETCH_SIZE`` and then
``--pmc WRITE_SIZE`` with ``--copy-bytes`` (a plain device copy of that many
bytes follows the timed region and calibrates the counters), then
``python bench.py --summarize-pmc FETCH_CSV WRITE_CSV`` writes
profiles/ffn_gate_up_gemm_traffic.json, which later runs report as
``roofline.traffic`` while the kernel source is unchanged.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s (route+plan+grouped FFN+combine), % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
DEFAULT_WORKLOAD = "c3_qwen3_235b_prefill"
GATE_UP_KERNEL = "ffn_persistent_kernel<0>"
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "ffn_gate_up_gemm_traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic_work(cfg):
    """FLOPs and HBM bytes each stage must move at minimum (per layer step)."""
    T, d, E, k, I = cfg.T, cfg.d, cfg.E, cfg.k, cfg.inter
    b = cfg.elem_bytes
    P = T * k
    f = {
        "gate_flop": 4.0 * T * d * E,
        "ffn_gate_up_flop": 4.0 * P * d * I,
        "ffn_down_flop": 2.0 * P * d * I,
        "shared_flop": 6.0 * T * d * cfg.shared_inter,
    }
    by = {
        "gate_topk": T * d * b + 2 * E * d * b + 12.0 * T * k,
        "permute_rows": T * d * b + P * d * b + 12.0 * P,
        "combine": P * d * b + 8.0 * P + T * d * b + (T * d * b if cfg.shared_inter else 0),
    }
    return f, by


def gate_up_roofline(cfg, active_experts, gu_ms):
    """Bound of the gate/up GEMM and its rate against that bound.  Algorithmic
    work: 4·P·d·I FLOP; algorithmic bytes: the weights of the experts that
    received pairs (2·I·d each), the unique token rows (T·d) and the SwiGLU
    output (P·I).  HBM-bound where FLOP / bytes is below the ridge
    (peak FLOP/s / peak bytes/s).  Returns (hbm_bound, achieved, peak, unit,
    bytes)."""
    flop = 4.0 * cfg.P * cfg.d * cfg.inter
    b = cfg.elem_bytes
    nbytes = active_experts * 2.0 * cfg.inter * cfg.d * b + cfg.T * cfg.d * b + cfg.P * cfg.inter * b
    hbm_bound = flop / nbytes < (PEAK_BF16_TFLOPS * 1e12) / (PEAK_HBM_GBS * 1e9)
    if hbm_bound:
        return True, nbytes / (gu_ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s", nbytes
    return False, flop / (gu_ms * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s", nbytes


def routing_stats(cfg, layer, idx_pred, home):
    """Reported alongside the throughput, from the step's device outputs:
    lookahead hit rate (fraction of the step's top-k assignments that the
    lookahead routing predicted) and spatial balance sum(L)/(G max L) of the
    per-rank loads without balancing (every pair at its expert's home) and
    after the split."""
    import torch
    idx = layer.idx.long()
    hit = (idx_pred.long()[:, :, None] == idx[:, None, :]).any(-1).sum().item() / idx.numel()
    per_expert = layer.counts.long().sum(0)
    static = torch.zeros(cfg.G, dtype=torch.long, device=idx.device).index_add_(0, home.long(), per_expert)
    split = layer.load.long()
    sp = lambda l: (l.sum() / (cfg.G * l.max().clamp(min=1))).item()  # noqa: E731
    return {"lookahead_hit": round(hit, 4), "spatial_static": round(sp(static), 4),
            "spatial_split": round(sp(split), 4)}


def cpu_baseline(cfg, li, w13, w2, shared, ntok):
    """The oracle as it stands, on the first ``ntok`` tokens of the workload."""
    import numpy as np
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    G, E, k = cfg.G, cfg.E, cfg.k
    t0 = time.perf_counter()
    h = li.h[:ntok]
    idx, w, gap, idx_next, _ = O.route(h, li.w_cur, li.b_cur, li.w_next, li.b_next, k, cfg.dtype)
    pred = O.route(li.h_prev[:ntok], li.w_cur, li.b_cur, None, None, k, cfg.dtype)[0]
    c, cn, cp = O.histogram(idx, G, E), O.histogram(idx_next, G, E), O.histogram(pred, G, E)
    rep_cur = O.plan(cp, li.home, G, E, cfg.N, cfg.L)
    O.plan(cn, li.home, G, E, cfg.N, cfg.L)
    hc, _ = O.split(c, li.home, rep_cur, G, E)
    off, perm, pos = O.permute(idx, li.home, rep_cur, hc, G, E)
    h64 = O.widen(h, cfg.dtype)
    out, _ = O.moe_via_groups(h64, idx, w, lambda e: (O.widen(w13[e], cfg.dtype), O.widen(w2[e], cfg.dtype)),
                              off, perm, pos, E)
    if shared is not None:
        out += O.swiglu(h64, O.widen(shared[0], cfg.dtype), O.widen(shared[1], cfg.dtype))
    dt = time.perf_counter() - t0
    return {"value": ntok / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {ntok} of {cfg.T} tokens of {cfg.name}, whole layer step (fp64), {dt:.1f} s"}


def time_two_stage(layer, args, K, stream, T):
    """The same step with MoE_local beside the split and the remote
    permutation: step time, its stages, and how much of the split stream's
    work stayed hidden under the local FFN."""
    import torch
    from routed_expert_ffn_gate_amd.layer import EVENTS_PER_STEP, TWO_STAGE_MARKS, HipEvents
    for _ in range(2):
        layer.step_two_stage(*args)
    torch.cuda.synchronize()
    EPS = EVENTS_PER_STEP
    ev = HipEvents(EPS * K + 2)
    ev.record(EPS * K, stream)
    for i in range(K):
        layer.step_two_stage(*args, events=ev, ev_base=EPS * i)
    ev.record(EPS * K + 1, stream)
    torch.cuda.synchronize()
    ms = ev.elapsed_ms(EPS * K, EPS * K + 1) / K
    st = {n: sum(ev.elapsed_ms(EPS * i + a, EPS * i + b) for i in range(K)) / K
          for n, (a, b) in TWO_STAGE_MARKS.items()}
    ev.close()
    side = st["split"] + st["permute_remote"]
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "stages_ms": {n: round(v, 4) for n, v in st.items()},
            "side_work_ms": round(side, 4), "exposed_ms": round(st["wait_remote"], 4),
            "hidden_ms": round(max(0.0, side - st["wait_remote"]), 4)}


def time_split_variants(layer, home, replica_cur, stream, reps=20):
    """Each split variant on this step's counts and placement: kernel time
    (HIP events around `reps` calls) and the spatial balance mean/max of the
    rank loads it leaves ("hash" = the even split, Relief with 0 passes)."""
    import torch
    from routed_expert_ffn_gate_amd import moelb as M
    from routed_expert_ffn_gate_amd.layer import HipEvents
    hc = torch.empty_like(layer.host_count)
    ld = torch.empty_like(layer.load)
    out = {}
    for name, code, passes in (("relief", M.MOELB_SPLIT_RELIEF, layer.passes),
                               ("no_reverse", M.MOELB_SPLIT_NO_REVERSE, layer.passes),
                               ("jacobi", M.MOELB_SPLIT_JACOBI, layer.passes),
                               ("libra_greedy", M.MOELB_SPLIT_LIBRA_GREEDY, layer.passes),
                               ("water_fill", M.MOELB_SPLIT_WATER_FILL, layer.passes),
                               ("hash", M.MOELB_SPLIT_RELIEF, 0)):
        ev = HipEvents(2)
        ev.record(0, stream)
        for _ in range(reps):
            M.moelb_split_variant(layer.counts, home, replica_cur, hc, ld, code, passes=passes, stream=stream)
        ev.record(1, stream)
        torch.cuda.synchronize()
        lf = ld.double()
        out[name] = {"us": round(1e3 * ev.elapsed_ms(0, 1) / reps, 2),
                     "spatial": round(float(lf.mean() / lf.max()), 4)}
        ev.close()
    return out


def time_graph(layer, tensors, K, W, stream):
    """The same step captured once in a HIP graph (torch.cuda.CUDAGraph; the
    lookahead stream forks and joins inside it by events) and replayed: the
    per-step time without per-launch host overhead and launch gaps."""
    import torch
    from routed_expert_ffn_gate_amd.layer import HipEvents
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.step(*tensors)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.step(*tensors)
    torch.cuda.synchronize()
    for _ in range(W):
        g.replay()
    ev = HipEvents(2)
    torch.cuda.synchronize()
    ev.record(0, stream)
    for _ in range(K):
        g.replay()
    ev.record(1, stream)
    torch.cuda.synchronize()
    ms = ev.elapsed_ms(0, 1) / K
    ev.close()
    del g
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(layer.T / (ms * 1e-3), 1)}


def time_stale_split(cfg, dev, stream, reps=20):
    """How often the split must be decided (Relief, "Failure of Existing
    Approaches"), over the workload's decode steps: each step plans its
    placement from its lookahead routing (the current router on the previous
    layer's input) and splits its actual counts fresh (Relief), evenly, and
    stale (the previous step's shares dealt by moelb_split_stale).  Reports
    the mean spatial balance sum(L)/(G max L) of each, the share of the fresh
    split's gain over the even split that the stale one gives up, and both
    kernels' times on the last step."""
    import torch
    from synth import workloads as W
    from routed_expert_ffn_gate_amd import moelb as M
    from routed_expert_ffn_gate_amd.layer import HipEvents, to_device
    S = cfg.steps
    if S < 2:
        return None
    G, E, k, T = cfg.G, cfg.E, cfg.k, cfg.T
    i32 = dict(dtype=torch.int32, device=dev)
    idx, idx_pred = torch.empty((T, k), **i32), torch.empty((T, k), **i32)
    wts = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts, counts_pred = torch.empty((G, E), **i32), torch.empty((G, E), **i32)
    rep = torch.empty((G, cfg.N), **i32)
    hc, hc_prev, hc_st = torch.empty((E, G), **i32), torch.empty((E, G), **i32), torch.empty((E, G), **i32)
    ld = torch.empty(G, **i32)
    sp = lambda l: float(l.double().sum() / (G * l.double().max().clamp(min=1)))  # noqa: E731
    acc = {"fresh": [], "even": [], "stale": [], "static": [], "loss_vs_even": []}
    for s in range(S):
        li = W.layer_inputs(cfg, step=s)
        up = lambda a: to_device(a, cfg.dtype, dev)  # noqa: E731
        h, h_prev, wc, bc, home = up(li.h), up(li.h_prev), up(li.w_cur), up(li.b_cur), up(li.home)
        M.moelb_gate_topk(h_prev, wc, bc, None, None, idx_pred, wts, stream=stream)
        M.moelb_histogram(idx_pred, G, counts_pred, stream=stream)
        M.moelb_plan(counts_pred, home, cfg.L, rep, stream=stream)
        M.moelb_gate_topk(h, wc, bc, None, None, idx, wts, stream=stream)
        M.moelb_histogram(idx, G, counts, stream=stream)
        M.moelb_split(counts, home, rep, hc, ld, passes=0, stream=stream)
        even = ld.clone()
        if s > 0:
            M.moelb_split_stale(counts, home, rep, hc_prev, hc_st, ld, stream=stream)
            stale = ld.clone()
        M.moelb_split(counts, home, rep, hc, ld, stream=stream)
        fresh = ld.clone()
        static = torch.zeros(G, dtype=torch.long, device=dev).index_add_(0, home.long(), counts.long().sum(0))
        if s > 0:
            acc["fresh"].append(sp(fresh))
            acc["even"].append(sp(even))
            acc["stale"].append(sp(stale))
            acc["static"].append(sp(static))
            f, e_, st = int(fresh.max()), int(even.max()), int(stale.max())
            if e_ > f:
                acc["loss_vs_even"].append((st - f) / (e_ - f))
        hc_prev.copy_(hc)
    ev = HipEvents(4)
    ev.record(0, stream)
    for _ in range(reps):
        M.moelb_split(counts, home, rep, hc, ld, stream=stream)
    ev.record(1, stream)
    ev.record(2, stream)
    for _ in range(reps):
        M.moelb_split_stale(counts, home, rep, hc_prev, hc_st, ld, stream=stream)
    ev.record(3, stream)
    torch.cuda.synchronize()
    out = {"steps": S - 1}
    for key, v in acc.items():
        out[key] = round(sum(v) / len(v), 4) if v else None
    out["relief_us"] = round(1e3 * ev.elapsed_ms(0, 1) / reps, 2)
    out["stale_us"] = round(1e3 * ev.elapsed_ms(2, 3) / reps, 2)
    ev.close()
    return out


def time_freebalance(cfg, tensors, K, W, stream, gather_rows=True, reps=20):
    """The same step with FreeBalance's expert swaps in place of replication
    (budget: the N replica slots as swaps per rank; gamma = 1 / mean rank
    load): step time, the balance its placement leaves, the swap count and
    the planner kernel's time."""
    import torch
    from routed_expert_ffn_gate_amd import moelb as M
    from routed_expert_ffn_gate_amd.layer import HipEvents, MoELayer
    h, h_prev, wc, bc, wn, bn, home, W13, W2, S13, S2 = tensors
    dev = h.device
    fl = MoELayer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.inter, cfg.G, cfg.N, cfg.L, cfg.dtype,
                  shared_inter=cfg.shared_inter, gather_rows=gather_rows, materialize_x=not gather_rows,
                  balancer="freebalance", fb_budget=cfg.N)
    home_cur = torch.empty((cfg.E,), dtype=torch.int32, device=dev)
    no_rep = torch.empty((cfg.G, 0), dtype=torch.int32, device=dev)
    fl.predict_placement(h_prev, wc, bc, home, home_cur)
    swaps = int(fl.n_swaps_next.item())  # the swaps that made this step's placement
    for _ in range(W):
        fl.step(h, wc, bc, wn, bn, home_cur, no_rep, W13, W2, S13, S2)
    ev = HipEvents(4)
    torch.cuda.synchronize()
    ev.record(0, stream)
    for _ in range(K):
        fl.step(h, wc, bc, wn, bn, home_cur, no_rep, W13, W2, S13, S2)
    ev.record(1, stream)
    torch.cuda.synchronize()
    ms = ev.elapsed_ms(0, 1) / K
    ld = fl.load.double()
    ho = torch.empty_like(home_cur)
    pl = torch.empty_like(fl.plan_load_next)
    ev.record(2, stream)
    for _ in range(reps):
        M.moelb_plan_swaps(fl.counts_next, home, ho, pl, tau=fl.fb_tau, gamma=fl.fb_gamma,
                           max_swaps_per_rank=fl.fb_budget, stream=stream)
    ev.record(3, stream)
    torch.cuda.synchronize()
    out = {"ms_per_step": round(ms, 4), "tokens_per_s": round(cfg.T / (ms * 1e-3), 1),
           "spatial": round(float(ld.mean() / ld.max()), 4), "swaps": swaps,
           "plan_us": round(1e3 * ev.elapsed_ms(2, 3) / reps, 2),
           "gamma": list(fl.fb_gamma), "swaps_per_rank_budget": fl.fb_budget}
    ev.close()
    del fl
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-tokens", type=int, default=32768)
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after the timed region, one plain device-to-device copy of this many bytes")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic summary from two rocprofv3 counter_collection.csv files")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--studies", action="store_true",
                    help="also measure the two-stage step, the split variants and FreeBalance's swaps "
                         "(reported beside the headline; their kernels then share the profile)")
    ap.add_argument("--rows", choices=["gather", "materialized"], default="gather",
                    help="gate/up GEMM reads h rows through the permutation, or a copied x_perm")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.workload, *args.summarize_pmc)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the expert-parallel ranks are simulated on a single MI355X; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from synth import workloads as W
    from routed_expert_ffn_gate_amd.layer import EVENTS_PER_STEP, HipEvents, MoELayer, stage_times_ms, to_device

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    cfg = W.config(args.workload)
    dev = torch.device("cuda:0")
    t0 = time.time()
    li = W.layer_inputs(cfg)
    w13, w2 = W.expert_weights_stacked(cfg, 1)
    shared = W.shared_weights(cfg)
    log(f"inputs generated in {time.time() - t0:.1f} s")
    up = lambda a: to_device(a, cfg.dtype, dev)  # noqa: E731
    h, h_prev = up(li.h), up(li.h_prev)
    wc, wn, bc, bn, home = up(li.w_cur), up(li.w_next), up(li.b_cur), up(li.b_next), up(li.home)
    W13, W2 = up(w13), up(w2)
    S13 = S2 = None
    if shared is not None:
        S13, S2 = up(shared[0]), up(shared[1])
    layer = MoELayer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.inter, cfg.G, cfg.N, cfg.L, cfg.dtype,
                     shared_inter=cfg.shared_inter, gather_rows=args.rows == "gather", materialize_x=True)
    replica_cur = torch.empty((cfg.G, cfg.N), dtype=torch.int32, device=dev)
    layer.predict_plan(h_prev, wc, bc, home, replica_cur)
    idx_pred = layer.idx_next.clone()  # the lookahead routing this step's plan was made from
    torch.cuda.synchronize()
    log(f"uploaded; workspace {layer.ws_ffn.numel() / 2**30:.2f} GiB")

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        layer.step(h, wc, bc, wn, bn, home, replica_cur, W13, W2, S13, S2)
    torch.cuda.synchronize()

    K = args.steps
    EPS = EVENTS_PER_STEP
    ev = HipEvents(EPS * K + 2)
    torch.cuda.synchronize()
    ev.record(EPS * K, stream)
    for i in range(K):
        layer.step(h, wc, bc, wn, bn, home, replica_cur, W13, W2, S13, S2, events=ev, ev_base=EPS * i)
    ev.record(EPS * K + 1, stream)
    torch.cuda.synchronize()
    total_ms = ev.elapsed_ms(EPS * K, EPS * K + 1)
    ms = total_ms / K
    stage = {}
    for i in range(K):
        for name, v in stage_times_ms(ev, EPS * i).items():
            stage[name] = stage.get(name, 0.0) + v / K
    sub = {n: stage.pop(n) for n in ("ffn_schedule", "ffn_gate_up_gemm", "ffn_down_gemm")}

    # the row-materialising permutation, timed on its own (the step reads rows
    # of h straight through the permutation instead)
    from routed_expert_ffn_gate_amd import moelb as M
    pe = HipEvents(2)
    pe.record(0, stream)
    reps = 5
    for _ in range(reps):
        M.moelb_permute(h, layer.idx, cfg.G, home, replica_cur, layer.host_count, layer.ws_perm, layer.group_off,
                        layer.perm, layer.pos, layer.x_perm)
    pe.record(1, stream)
    permute_rows_ms = pe.elapsed_ms(0, 1) / reps

    balance = routing_stats(cfg, layer, idx_pred, home)
    studies = {}
    if args.studies:
        studies["two_stage"] = time_two_stage(layer, (h, wc, bc, wn, bn, home, replica_cur, W13, W2, S13, S2), K,
                                              stream, cfg.T)
        studies["split_variants"] = time_split_variants(layer, home, replica_cur, stream)
        studies["freebalance"] = time_freebalance(cfg, (h, h_prev, wc, bc, wn, bn, home, W13, W2, S13, S2), K,
                                                  args.warmup, stream, gather_rows=args.rows == "gather")
        studies["stale_split"] = time_stale_split(cfg, dev, stream)
        studies["graph"] = time_graph(layer, (h, wc, bc, wn, bn, home, replica_cur, W13, W2, S13, S2), K,
                                      args.warmup, stream)
    f, by = algorithmic_work(cfg)
    total_flop = f["gate_flop"] + f["ffn_gate_up_flop"] + f["ffn_down_flop"] + f["shared_flop"]
    tokens_per_s = cfg.T / (ms * 1e-3)
    gu_ms = sub["ffn_gate_up_gemm"]
    active = int((layer.counts.long().sum(0) > 0).sum().item())
    gu_hbm_bound, achieved, peak, unit, gu_bytes = gate_up_roofline(cfg, active, gu_ms)
    hbm = {
        "gate_topk": by["gate_topk"] / (stage["gate_topk"] * 1e-3) / 1e9,
        "permute_rows": by["permute_rows"] / (permute_rows_ms * 1e-3) / 1e9,
        "combine": by["combine"] / (stage["combine"] * 1e-3) / 1e9,
    }
    traffic = None
    if os.path.exists(TRAFFIC_JSON):
        with open(TRAFFIC_JSON) as fh:
            tr = json.load(fh)
        if tr.get("workload") == cfg.name and tr.get("kernel_source_sha") == _kernel_sha():
            traffic = tr.get("bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded; shapes of the workload, random-init router and experts)",
        "config": {"workload": cfg.name, "tokens": cfg.T, "hidden": cfg.d, "experts": cfg.E, "top_k": cfg.k,
                   "inter": cfg.inter, "shared_inter": cfg.shared_inter, "virtual_ranks": cfg.G,
                   "replica_slots": cfg.N, "locality_imports": cfg.L, "relief_passes": 12,
                   "ffn_rows": args.rows},
        "mfma_frac_layer": round(total_flop / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 4),
        "roofline": {"bound": "hbm" if gu_hbm_bound else "mfma",
                     "kernel": (GATE_UP_KERNEL if cfg.dtype == "bf16" else "ffn_simt_kernel<0>") +
                     " (gate/up GEMM + SwiGLU)",
                     "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "flop_per_launch": f["ffn_gate_up_flop"], "bytes_per_launch": gu_bytes,
                     "avg_launch_ms": round(gu_ms, 4)},
        "stages_ms": {k_: round(v, 4) for k_, v in {**stage, **sub, "permute_rows": permute_rows_ms}.items()},
        "hbm_frac": {k_: round(v / PEAK_HBM_GBS, 4) for k_, v in hbm.items()},
        "routing": balance,
        **studies,
        "ffn_mfma_frac": round((f["ffn_gate_up_flop"] + f["ffn_down_flop"]) /
                               ((sub["ffn_gate_up_gemm"] + sub["ffn_down_gemm"]) * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
                               4),
    }
    if args.copy_bytes > 0:
        # plain copy of known size: the counters' calibration in a PMC run
        n = args.copy_bytes // 4
        src = torch.ones(n, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_bytes"] = n * 4
        del src, dst
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(cfg, li, w13, w2, shared, args.cpu_tokens)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def _read_pmc(path, counter):
    import csv
    rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
    return rows


def summarize_pmc(workload, fetch_csv, write_csv):
    """Per-dispatch HBM-side bytes of the gate/up GEMM from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by the factor that maps the same
    counter on the largest plain copy dispatch to the bytes it must move."""
    out = {"workload": workload, "kernel": GATE_UP_KERNEL, "kernel_source_sha": _kernel_sha()}
    for key, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        rows = _read_pmc(path, counter)
        gu = [float(r["Counter_Value"]) for r in rows if GATE_UP_KERNEL in r["Kernel_Name"]]
        cp = [r for r in rows if "copy" in r["Kernel_Name"].lower()]
        if not gu or not cp:
            raise SystemExit(f"{path}: no gate/up or copy dispatch with {counter}")
        big = max(cp, key=lambda r: float(r["Counter_Value"]))
        out[f"{key}_kib_per_dispatch"] = sum(gu) / len(gu)
        out[f"{key}_dispatches"] = len(gu)
        out[f"{key}_copy_kib"] = float(big["Counter_Value"])
        out[f"{key}_copy_kernel"] = big["Kernel_Name"]
    out["note"] = ("copy of copy_bytes moves copy_bytes read + copy_bytes written; factor = copy_bytes / "
                   "(counter KiB x 1024) per counter")
    cb = int(os.environ.get("COPY_BYTES", "0"))
    if cb <= 0:
        raise SystemExit("set COPY_BYTES to the --copy-bytes of the PMC runs")
    out["copy_bytes"] = cb
    f_fetch = cb / (out["fetch_copy_kib"] * 1024.0)
    f_write = cb / (out["write_copy_kib"] * 1024.0)
    out["fetch_factor"], out["write_factor"] = f_fetch, f_write
    out["bytes_per_launch"] = (out["fetch_kib_per_dispatch"] * 1024.0 * f_fetch +
                               out["write_kib_per_dispatch"] * 1024.0 * f_write)
    with open(TRAFFIC_JSON, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def _kernel_sha():
    import hashlib
    p = os.path.join(ROOT, "routed_expert_ffn_gate_amd", "csrc", "grouped_ffn.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


if __name__ == "__main__":
    main()
