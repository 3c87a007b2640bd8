#!/usr/bin/env python3
"""MoE-layer throughput of the routing-and-balancing hot path on one MI355X.

One step = one whole layer step on one batch: gate + lookahead gate, two
histograms, plan for the next layer, Relief split, permutation, grouped
SwiGLU FFN (+ shared expert where the workload has one) and combine.  Inputs
are seeded synthetic tensors of the workload's shapes, resident in HBM before
the timed region.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload NAME]

Counters: one kernel-trace run and three counter runs (FETCH_SIZE;
WRITE_SIZE; MFMA operations and busy cycles) of the same command with
``--copy-bytes`` (a plain device copy of that many bytes follows the timed
region and calibrates the traffic counters), then ``python bench.py
--summarize-profile DIR KT_JSON`` writes profiles/kernels_<workload>.md and
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


def host_cpu():
    """CPU model, the cores this process may run on, and the BLAS threads."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    return model, cores, blas


def cpu_baseline(cfg, li, w13, w2, shared, ntok):
    """The oracle as it stands, on the first ``ntok`` tokens of the workload:
    the whole layer step in fp64 (route with lookahead, prologue routing,
    three histograms, both plans, split, permutation, grouped FFN and
    combine), each stage timed."""
    from oracle import moe_oracle as O
    model, cores, blas = host_cpu()
    G, E, k = cfg.G, cfg.E, cfg.k
    st = {}
    t_all = time.perf_counter()

    def lap(name, t0):
        st[name] = round(time.perf_counter() - t0, 3)
        return time.perf_counter()

    t = time.perf_counter()
    h = li.h[:ntok]
    idx, w, gap, idx_next, _ = O.route(h, li.w_cur, li.b_cur, li.w_next, li.b_next, k, cfg.dtype)
    pred = O.route(li.h_prev[:ntok], li.w_cur, li.b_cur, None, None, k, cfg.dtype)[0]
    t = lap("gate_topk", t)
    c, cn, cp = O.histogram(idx, G, E), O.histogram(idx_next, G, E), O.histogram(pred, G, E)
    t = lap("histogram", t)
    rep_cur = O.plan(cp, li.home, G, E, cfg.N, cfg.L)
    O.plan(cn, li.home, G, E, cfg.N, cfg.L)
    t = lap("plan", t)
    hc, _ = O.split(c, li.home, rep_cur, G, E)
    t = lap("split", t)
    off, perm, pos = O.permute(idx, li.home, rep_cur, hc, G, E)
    t = lap("permute", t)
    h64 = O.widen(h, cfg.dtype)
    out, _ = O.moe_via_groups(h64, idx, w, lambda e: (O.widen(w13[e], cfg.dtype), O.widen(w2[e], cfg.dtype)),
                              off, perm, pos, E)
    if shared is not None:
        out += O.swiglu(h64, O.widen(shared[0], cfg.dtype), O.widen(shared[1], cfg.dtype))
    lap("grouped_ffn_combine", t)
    dt = time.perf_counter() - t_all
    return {"value": ntok / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {ntok} of {cfg.T} tokens of {cfg.name}, whole layer step (fp64), {dt:.1f} s",
            "cpu_model": model, "blas_threads": int(blas), "stage_s": st}


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
                               ("proportional", M.MOELB_SPLIT_PROPORTIONAL, layer.passes),
                               ("hash", M.MOELB_SPLIT_RELIEF, 0)):
        if code == M.MOELB_SPLIT_PROPORTIONAL and layer.G > 16:
            continue  # exact shares for at most 16 hosts per expert
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


def time_freebalance(cfg, tensors, K, W, stream, gather_rows=True, reps=20, packed=False):
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
                  balancer="freebalance", fb_budget=cfg.N, packed_weights=packed)
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


def _median(v):
    v = sorted(v)
    n = len(v)
    return 0.0 if n == 0 else (v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2]))


def prepare_units(cfg, layer, dev):
    """The layer steps a timed run cycles through, inputs resident in HBM: the
    workload's one layer; or each of the drift workload's layers (its own
    router and experts; layer 1's plan from the prologue's lookahead, layer
    l+1's from layer l's lookahead, made by the step itself); or each decode
    step (re-drawn inputs, fixed weights, plan from its own predicted
    routing).  Each unit keeps its placement, split schedule and the routing
    its plan was made from."""
    import torch
    from synth import workloads as W
    from routed_expert_ffn_gate_amd.layer import to_device
    from routed_expert_ffn_gate_amd.layer import pack_expert_weights
    up = lambda a: to_device(a, cfg.dtype, dev)  # noqa: E731

    def upw(a):
        """Expert weights to the device, packed once for the FFN's weight
        streams when the layer takes them so (model-load work, outside every
        timed region)."""
        t = up(a)
        if not layer.ffn_opt:
            return t
        p = pack_expert_weights(t)
        torch.cuda.synchronize()
        del t
        return p

    home = up(W.resident_home(cfg))
    shared = W.shared_weights(cfg)
    S13, S2 = (upw(shared[0]), upw(shared[1])) if shared is not None else (None, None)
    units = []

    def unit(name, li, W13, W2):
        return {"name": name, "li": li, "h": up(li.h), "h_prev": up(li.h_prev), "wc": up(li.w_cur),
                "bc": up(li.b_cur), "wn": up(li.w_next), "bn": up(li.b_next), "W13": W13, "W2": W2}

    def prologue(u):
        u["replica"] = torch.empty((cfg.G, cfg.N), dtype=torch.int32, device=dev)
        layer.predict_plan(u["h_prev"], u["wc"], u["bc"], home, u["replica"])
        u["sched"] = layer.sched_cur.clone()
        u["idx_pred"] = layer.idx_next.clone()

    if cfg.layers > 1:
        hs = W.hidden_states(cfg, cfg.layers)
        for l in range(1, cfg.layers + 1):
            w13, w2 = W.expert_weights_stacked(cfg, l)
            units.append(unit(f"layer{l}", W.layer_inputs(cfg, l, 0, hs=hs), upw(w13), upw(w2)))
            del w13, w2
        prologue(units[0])
        for a, b in zip(units, units[1:]):
            layer.step(a["h"], a["wc"], a["bc"], a["wn"], a["bn"], home, a["replica"], a["W13"], a["W2"], S13, S2,
                       sched=a["sched"])
            b["idx_pred"] = layer.idx_next.clone()
            b["replica"] = layer.advance().clone()
            b["sched"] = layer.sched_cur.clone()
    else:
        w13, w2 = W.expert_weights_stacked(cfg, 1)
        W13, W2 = upw(w13), upw(w2)
        del w13, w2
        for st in range(cfg.steps):
            u = unit(f"step{st}" if cfg.steps > 1 else "layer1", W.layer_inputs(cfg, 1, st), W13, W2)
            prologue(u)
            units.append(u)
    torch.cuda.synchronize()
    return units, home, S13, S2


def weights_packable(cfg):
    """moelb_pack_weights' and the packed FFN's shape rules."""
    return (cfg.dtype == "bf16" and cfg.d % 64 == 0 and cfg.inter % 64 == 0 and
            (not cfg.shared_inter or cfg.shared_inter % 64 == 0))


def run_unit(layer, u, home, S13, S2, **kw):
    return layer.step(u["h"], u["wc"], u["bc"], u["wn"], u["bn"], home, u["replica"], u["W13"], u["W2"], S13, S2,
                      sched=u["sched"], **kw)


def rank_times(layer, u, home, S13, S2, stream, reps=5):
    """One virtual rank's share of the grouped FFN (its local and remote
    groups), timed alone for every rank on this step's permutation: t_r
    (median of ``reps`` launches), the slowest, and the time-spatial balance
    mean/max."""
    from routed_expert_ffn_gate_amd import moelb as M
    from routed_expert_ffn_gate_amd.layer import HipEvents
    run_unit(layer, u, home, S13, S2)
    x = u["h"] if layer.gather_rows else layer.x_perm
    kw = dict(gather=layer.perm, gather_k=layer.k) if layer.gather_rows else {}
    ev = HipEvents(2 * reps)
    t = []
    for r in range(layer.G):
        for i in range(reps):
            ev.record(2 * i, stream)
            M.moelb_grouped_ffn_stages(M.MOELB_FFN_ALL | layer.ffn_opt, x, layer.P, layer.group_off, layer.E,
                                       u["W13"], u["W2"], layer.ws_ffn, layer.y, G=layer.G, rank=r, stream=stream,
                                       **kw)
            ev.record(2 * i + 1, stream)
        t.append(_median([ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(reps)]))
    ev.close()
    return t


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed layer steps (default 20; 24 for workloads of 8 layers or decode steps)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-tokens", type=int, default=32768)
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after the timed region, one plain device-to-device copy of this many bytes")
    ap.add_argument("--summarize-profile", nargs=2, metavar=("PROF_DIR", "BENCH_JSON"),
                    help="write profiles/kernels_<workload>.md from a kernel-trace run and three counter runs "
                         "(PROF_DIR/kt, pmc_f, pmc_w, pmc_m) and the bench line of the kernel-trace run")
    ap.add_argument("--summarize-runs", nargs="+", metavar="ARG",
                    help="OUT_NAME COMMAND JSON...: write profiles/OUT_NAME.md from bench result lines")
    ap.add_argument("--summarize-counters", nargs=1, metavar="PROF_DIR",
                    help="write profiles/counters_<workload>.md from the stall counter runs PROF_DIR/pmc_s "
                         "(LDS and wait counters) and PROF_DIR/pmc_t (texture unit and issue counters)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rank-times", action="store_true",
                    help="skip the per-virtual-rank FFN timing (for counter runs)")
    ap.add_argument("--studies", action="store_true",
                    help="also measure the two-stage step, the split variants and FreeBalance's swaps "
                         "(reported beside the headline; their kernels then share the profile)")
    ap.add_argument("--split-overlap", choices=["auto", "on", "off"], default="auto",
                    help="the split beside the local half of the permutation (auto: where the permutation is "
                         "not one launch anyway)")
    ap.add_argument("--weights", choices=["packed", "row-major"], default="packed",
                    help="expert weights packed once by moelb_pack_weights (where the shape allows), or row-major")
    ap.add_argument("--rows", choices=["gather", "materialized"], default="gather",
                    help="gate/up GEMM reads h rows through the permutation, or a copied x_perm")
    args = ap.parse_args()
    if args.summarize_profile:
        summarize_profile(args.workload, *args.summarize_profile)
        return
    if args.summarize_counters:
        summarize_counters(args.workload, args.summarize_counters[0])
        return
    if args.summarize_runs:
        summarize_runs(args.summarize_runs[2:], args.summarize_runs[0], args.summarize_runs[1])
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the expert-parallel ranks are simulated on a single MI355X; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from synth import workloads as W
    from routed_expert_ffn_gate_amd import moelb as M
    from routed_expert_ffn_gate_amd.layer import EVENTS_PER_STEP, HipEvents, MoELayer, stage_times_ms

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    cfg = W.config(args.workload)
    dev = torch.device("cuda:0")
    t0 = time.time()
    packed = args.weights == "packed" and weights_packable(cfg)
    layer = MoELayer(cfg.T, cfg.d, cfg.E, cfg.k, cfg.inter, cfg.G, cfg.N, cfg.L, cfg.dtype,
                     shared_inter=cfg.shared_inter, gather_rows=args.rows == "gather", materialize_x=True,
                     packed_weights=packed,
                     overlap_split=None if args.split_overlap == "auto" else args.split_overlap == "on")
    units, home, S13, S2 = prepare_units(cfg, layer, dev)
    n_units = len(units)
    u0 = units[0]
    log(f"{n_units} layer step(s) prepared in {time.time() - t0:.1f} s; "
        f"FFN workspace {layer.ws_ffn.numel() / 2**30:.2f} GiB")

    stream = torch.cuda.current_stream()
    K = args.steps if args.steps is not None else (20 if n_units == 1 else 3 * n_units)
    for i in range(max(args.warmup, n_units)):
        run_unit(layer, units[i % n_units], home, S13, S2)
    torch.cuda.synchronize()

    # the timed region: K layer steps, one event between consecutive steps
    tev = HipEvents(K + 1)
    torch.cuda.synchronize()
    for i in range(K):
        tev.record(i, stream)
        run_unit(layer, units[i % n_units], home, S13, S2)
    tev.record(K, stream)
    torch.cuda.synchronize()
    total_ms = tev.elapsed_ms(0, K)
    ms = total_ms / K
    step_ms = [tev.elapsed_ms(i, i + 1) for i in range(K)]
    tev.close()
    # the stage breakdown: the same K steps again, with a mark around every
    # stage (the marks cost a few microseconds each, so they stay out of the
    # timed region)
    EPS = EVENTS_PER_STEP
    ev = HipEvents(EPS * K)
    torch.cuda.synchronize()
    for i in range(K):
        run_unit(layer, units[i % n_units], home, S13, S2, events=ev, ev_base=EPS * i)
    torch.cuda.synchronize()
    per_step = [stage_times_ms(ev, EPS * i) for i in range(K)]
    marked_ms = [ev.elapsed_ms(EPS * i, EPS * i + 7) for i in range(K)]
    ev.close()
    names = list(per_step[0])
    mean_st = {n: sum(p[n] for p in per_step) / K for n in names}
    med_st = {n: _median([p[n] for p in per_step]) for n in names}

    # the row-materialising permutation, timed on its own (the step reads rows
    # of h straight through the permutation instead)
    run_unit(layer, u0, home, S13, S2)
    pe = HipEvents(2)
    pe.record(0, stream)
    reps = 5
    for _ in range(reps):
        M.moelb_permute(u0["h"], layer.idx, cfg.G, home, u0["replica"], layer.host_count, layer.ws_perm,
                        layer.group_off, layer.perm, layer.pos, layer.x_perm)
    pe.record(1, stream)
    permute_rows_ms = pe.elapsed_ms(0, 1) / reps
    # the split when the schedule does not match the placement (placement
    # changed since the schedule was made): the kernel colours the transfers
    pe.record(0, stream)
    for _ in range(20):
        M.moelb_split_scheduled(layer.counts, home, u0["replica"], None, layer.host_count, layer.load,
                                passes=layer.passes, stream=stream)
    pe.record(1, stream)
    split_unscheduled_ms = pe.elapsed_ms(0, 1) / 20
    pe.close()

    # per unit: routing quality, balance, stage medians, per-rank FFN times
    f, by = algorithmic_work(cfg)
    unit_rows = []
    gu_bytes_time = [0.0, 0.0]
    for j, u in enumerate(units):
        run_unit(layer, u, home, S13, S2)
        torch.cuda.synchronize()
        r = routing_stats(cfg, layer, u["idx_pred"], home)
        # the plan alone (even split of its pools) and the plan + split, against no balancing
        M.moelb_split(layer.counts, home, u["replica"], layer.host_count, layer.load, passes=0, stream=stream)
        ld = layer.load.double()
        r["spatial_plan_even"] = round(float(ld.sum() / (cfg.G * ld.max().clamp(min=1))), 4)
        r["improved"] = r["spatial_split"] > r["spatial_static"]
        active = int((layer.counts.long().sum(0) > 0).sum().item())
        r["active_experts"] = active
        idx_steps = [i for i in range(K) if i % n_units == j]
        st = {n: round(_median([per_step[i][n] for i in idx_steps]), 4) for n in names}
        gu = [per_step[i]["ffn_gate_up_gemm"] for i in idx_steps]
        _, _, _, _, gbytes = gate_up_roofline(cfg, active, 1.0)
        gu_bytes_time[0] += gbytes * len(gu)
        gu_bytes_time[1] += sum(gu)
        row = {"name": u["name"], "ms_median": round(_median([step_ms[i] for i in idx_steps]), 4),
               "ms_median_marked": round(_median([marked_ms[i] for i in idx_steps]), 4),
               "stages_ms": st, **r}
        if not args.no_rank_times:
            t_r = rank_times(layer, u, home, S13, S2, stream)
            t_max = max(t_r)
            t_split = st["split"]
            t_plan = st["side_histogram_plan"]
            row["rank_ffn_ms"] = [round(x, 4) for x in t_r]
            row["rank_ffn_max_ms"] = round(t_max, 4)
            row["time_spatial"] = round(sum(t_r) / (len(t_r) * t_max), 4)
            # Relief "Effective Utilization Metric": spatial / (1 + T_solve / T_moe),
            # T_moe = the slowest rank's FFN, T_solve = the per-step split
            # (and, second form, the plan made beside the previous step as well)
            row["u_eff"] = round(r["spatial_split"] / (1.0 + t_split / t_max), 4)
            row["u_eff_with_plan"] = round(r["spatial_split"] / (1.0 + (t_split + t_plan) / t_max), 4)
        unit_rows.append(row)
    torch.cuda.synchronize()

    studies = {}
    if args.studies:
        tensors = (u0["h"], u0["wc"], u0["bc"], u0["wn"], u0["bn"], home, u0["replica"], u0["W13"], u0["W2"], S13,
                   S2)
        layer.sched_cur.copy_(u0["sched"])
        studies["two_stage"] = time_two_stage(layer, tensors, K, stream, cfg.T)
        run_unit(layer, u0, home, S13, S2)
        studies["split_variants"] = time_split_variants(layer, home, u0["replica"], stream)
        studies["freebalance"] = time_freebalance(cfg, (u0["h"], u0["h_prev"], u0["wc"], u0["bc"], u0["wn"],
                                                        u0["bn"], home, u0["W13"], u0["W2"], S13, S2), K,
                                                  args.warmup, stream, gather_rows=args.rows == "gather",
                                                  packed=packed)
        studies["stale_split"] = time_stale_split(cfg, dev, stream)
        studies["graph"] = time_graph(layer, tensors, K, args.warmup, stream)

    total_flop = f["gate_flop"] + f["ffn_gate_up_flop"] + f["ffn_down_flop"] + f["shared_flop"]
    tokens_per_s = cfg.T / (ms * 1e-3)
    gu_ms = mean_st["ffn_gate_up_gemm"]
    gu_hbm_bound, _, peak, unit, _ = gate_up_roofline(cfg, unit_rows[0]["active_experts"], gu_ms)
    gu_bytes = gu_bytes_time[0] / K
    if gu_hbm_bound:
        achieved = gu_bytes_time[0] / (gu_bytes_time[1] * 1e-3) / 1e9
    else:
        achieved = f["ffn_gate_up_flop"] / (gu_ms * 1e-3) / 1e12
    hbm = {
        "gate_topk": by["gate_topk"] / (med_st["gate_topk"] * 1e-3) / 1e9,
        "permute_rows": by["permute_rows"] / (permute_rows_ms * 1e-3) / 1e9,
        "combine": by["combine"] / (med_st["combine"] * 1e-3) / 1e9,
    }
    traffic = None
    if os.path.exists(TRAFFIC_JSON):
        with open(TRAFFIC_JSON) as fh:
            tr = _traffic_records(json.load(fh)).get(cfg.name, {})
        if (tr.get("workload") == cfg.name and tr.get("kernel_source_sha") == _kernel_sha() and
                tr.get("ffn_weights", "row-major") == ("packed" if packed else "row-major")):
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
                   "layer_steps_cycled": n_units, "ffn_rows": args.rows,
                   "ffn_weights": "packed" if packed else "row-major", "split_overlap": layer.overlap_split},
        "ms_per_step_median": round(_median(step_ms), 4),
        "ms_per_step_marked_median": round(_median(marked_ms), 4),
        "mfma_frac_layer": round(total_flop / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 4),
        "roofline": {"bound": "hbm" if gu_hbm_bound else "mfma",
                     "kernel": (GATE_UP_KERNEL if cfg.dtype == "bf16" else "ffn_simt_kernel<0>") +
                     " (gate/up GEMM + SwiGLU)",
                     "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "flop_per_launch": f["ffn_gate_up_flop"], "bytes_per_launch": gu_bytes,
                     "avg_launch_ms": round(gu_ms, 4)},
        "stages_ms": {k_: round(v, 4) for k_, v in {**med_st, "permute_rows": permute_rows_ms,
                                                       "split_unscheduled": split_unscheduled_ms}.items()},
        "stages_ms_mean": {k_: round(v, 4) for k_, v in mean_st.items()},
        "hbm_frac": {k_: round(v / PEAK_HBM_GBS, 4) for k_, v in hbm.items()},
        "ffn_mfma_frac": round((f["ffn_gate_up_flop"] + f["ffn_down_flop"]) /
                               ((med_st["ffn_gate_up_gemm"] + med_st["ffn_down_gemm"]) * 1e-3) /
                               (PEAK_BF16_TFLOPS * 1e12), 4),
        "routing": {k_: v for k_, v in unit_rows[0].items()
                    if k_ in ("lookahead_hit", "spatial_static", "spatial_plan_even", "spatial_split",
                              "active_experts")},
        "balance": {k_: v for k_, v in unit_rows[0].items()
                    if k_ in ("rank_ffn_ms", "rank_ffn_max_ms", "time_spatial", "u_eff", "u_eff_with_plan")},
        **studies,
    }
    if n_units > 1:
        result["units"] = unit_rows
        result["units_mean"] = {
            key: round(sum(float(r_[key]) for r_ in unit_rows) / n_units, 4)
            for key in ("ms_median", "lookahead_hit", "spatial_static", "spatial_plan_even", "spatial_split",
                        "u_eff", "time_spatial") if key in unit_rows[0]}
        result["units_mean"]["improved_share"] = round(sum(r_["improved"] for r_ in unit_rows) / n_units, 4)
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
        w13, w2 = W.expert_weights_stacked(cfg, u0["li"].layer)
        result["cpu_baseline"] = cpu_baseline(cfg, u0["li"], w13, w2, W.shared_weights(cfg), args.cpu_tokens)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def _short_kernel(name):
    """Kernel name without 'void', the anonymous namespace and the argument list."""
    n = name.replace("void ", "").replace("(anonymous namespace)::", "")
    depth = 0
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return n[:i]
    return n


def _dispatches(path, counter=None):
    """Per-dispatch rows of a rocprofv3 CSV (kernel trace or counter
    collection): (kernel, duration s, counter value or None)."""
    import csv
    out = []
    for r in csv.DictReader(open(path)):
        if counter is not None and r.get("Counter_Name") != counter:
            continue
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        out.append((_short_kernel(r["Kernel_Name"]), dur, float(r["Counter_Value"]) if counter else None))
    return out


# the row-copying permutation is the same kernel as the index-only one: a
# launch is a row copy if it writes more than ROWS_WRITE_FACTOR times the
# index bytes (12 per pair) in the WRITE_SIZE run, whose launches come in the
# same order as in every other run of the same command
ROWS_WRITE_FACTOR = 4.0


def _rows_launches(write_rows, fw, pairs):
    """For each rank_scatter_kernel launch in order: does it copy rows?"""
    return [v * 1024 * fw > ROWS_WRITE_FACTOR * 12.0 * pairs
            for n, _, v in write_rows if n.startswith("rank_scatter_kernel")]


# kernels of the bench's input preparation (weights packed once, as at model
# load), listed apart in the profile table
SETUP_KERNELS = ("pack_weights_kernel",)


FFN_GEMM_KERNELS = ("ffn_persistent_kernel", "ffn_skinny_kernel", "ffn_mfma_dma_kernel", "ffn_mfma_kernel",
                    "ffn_simt_kernel")


def _shared_launches(mops_rows, f):
    """For each FFN GEMM launch in order, per kernel name: is it the shared
    expert's (executed MFMA work under half the routed GEMM's)?"""
    import collections
    flags = collections.defaultdict(list)
    for n, _, v in mops_rows:
        if n.startswith(FFN_GEMM_KERNELS):
            routed = f["ffn_gate_up_flop"] if n.endswith("<0>") else f["ffn_down_flop"]
            flags[n].append(v * 512 < 0.5 * routed)
    return flags


def _kernel_key(name, rows_flag):
    if name.startswith("rank_scatter_kernel"):
        return name + (" (rows)" if rows_flag else " (indices)")
    return name


def kernel_work(cfg, active):
    """Algorithmic work per launch of the step's kernels: (bound, amount, unit)
    with bytes for HBM-bound kernels and FLOP for MFMA-bound ones."""
    T, d, E, k, I, G = cfg.T, cfg.d, cfg.E, cfg.k, cfg.inter, cfg.G
    b = cfg.elem_bytes
    P = T * k
    f, by = algorithmic_work(cfg)
    return {
        "gate_topk_dma_kernel": ("hbm", by["gate_topk"], "B"),
        "histogram_kernel": ("hbm", 4.0 * P + 4.0 * G * E, "B"),
        "count_kernel": ("hbm", 4.0 * P, "B"),
        "rank_scatter_kernel (indices)": ("hbm", 12.0 * P, "B"),
        "rank_scatter_kernel (rows)": ("hbm", by["permute_rows"], "B"),
        "ffn_persistent_kernel<0>": ("mfma", f["ffn_gate_up_flop"], "FLOP"),
        "ffn_persistent_kernel<1>": ("mfma", f["ffn_down_flop"], "FLOP"),
        "ffn_skinny_kernel<0>": ("mfma", f["ffn_gate_up_flop"], "FLOP"),
        "ffn_skinny_kernel<1>": ("mfma", f["ffn_down_flop"], "FLOP"),
        "combine_kernel": ("hbm", by["combine"], "B"),
        # the shared expert's GEMMs (one group of all T tokens), after the
        # routed ones so that plain names match those first
        "ffn_persistent_kernel<0> (shared expert)": ("mfma", 4.0 * T * d * cfg.shared_inter, "FLOP"),
        "ffn_persistent_kernel<1> (shared expert)": ("mfma", 2.0 * T * d * cfg.shared_inter, "FLOP"),
        "_ffn_bytes": (active * 2.0 * I * d * b + T * d * b + P * I * b, P * I * b + active * d * I * b + P * d * b),
    }


def summarize_profile(workload, prof_dir, bench_json):
    """Per-kernel table from one kernel-trace run and three counter runs of
    the same command (FETCH_SIZE, WRITE_SIZE, and the MFMA/clock counters),
    each in ``prof_dir`` (kt/, pmc_f/, pmc_w/, pmc_m/).  FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) are scaled by the factor that maps the same
    counter on the largest plain copy dispatch (copy_bytes each way) to its
    known bytes.  Writes profiles/kernels_<workload>.md and, for the gate/up
    GEMM, the traffic record bench.py reports as roofline.traffic."""
    import collections
    from synth import workloads as W
    cfg = W.config(workload)
    res = json.load(open(bench_json))
    active = res["routing"]["active_experts"]
    cb = int(res["copy_bytes"])
    kt = _dispatches(os.path.join(prof_dir, "kt", "kt_kernel_trace.csv"))
    pf = os.path.join(prof_dir, "pmc_f", "p_counter_collection.csv")
    pw = os.path.join(prof_dir, "pmc_w", "p_counter_collection.csv")
    pm = os.path.join(prof_dir, "pmc_m", "p_counter_collection.csv")
    fetch, write = _dispatches(pf, "FETCH_SIZE"), _dispatches(pw, "WRITE_SIZE")
    mops, grbm = _dispatches(pm, "SQ_INSTS_VALU_MFMA_MOPS_BF16"), _dispatches(pm, "GRBM_GUI_ACTIVE")
    mbusy = _dispatches(pm, "SQ_VALU_MFMA_BUSY_CYCLES")
    simds = 4 * int(res.get("compute_units", 256))
    copy_f = max(v for n, _, v in fetch if "copyBuffer" in n)
    copy_w = max(v for n, _, v in write if "copyBuffer" in n)
    ff, fw = cb / (copy_f * 1024.0), cb / (copy_w * 1024.0)

    is_rows = _rows_launches(write, fw, cfg.T * cfg.k)
    is_shared = _shared_launches(mops, algorithmic_work(cfg)[0]) if cfg.shared_inter else {}

    def per_kernel(rows):
        agg = collections.defaultdict(list)
        i = 0
        seen = collections.Counter()
        for n, dur, v in rows:
            flag = False
            if n.startswith("rank_scatter_kernel"):
                flag = is_rows[i] if i < len(is_rows) else False
                i += 1
            key = _kernel_key(n, flag)
            if n in is_shared:
                j = seen[n]
                seen[n] += 1
                if j < len(is_shared[n]) and is_shared[n][j]:
                    key = n + " (shared expert)"
            agg[key].append((dur, v))
        return agg

    KT, F, Wr, MO, GR, MB = (per_kernel(x) for x in (kt, fetch, write, mops, grbm, mbusy))
    work = kernel_work(cfg, active)
    ffn_bytes = work.pop("_ffn_bytes")
    f, _ = algorithmic_work(cfg)
    lines = [f"# Kernels of one layer step, {workload}, one MI355X", "",
             "Durations: rocprofv3 kernel trace (average per launch). Traffic: FETCH_SIZE and WRITE_SIZE per "
             f"launch, each scaled by the factor that maps the counter on a plain {cb >> 20} MiB device copy to "
             f"the bytes it moves (FETCH x{ff:.4f}, WRITE x{fw:.4f}). MFMA: SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 "
             "FLOP (executed, padding included) per launch, over the launch's duration in the counter run. "
             "MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES per launch over the launch's SIMD cycles (GRBM_GUI_ACTIVE / 8 "
             f"XCDs x {simds} SIMDs). "
             "Clock: GRBM_GUI_ACTIVE per launch / duration / 8 XCDs, for launches of 200 µs or more (counter "
             "run; the profiler slows long kernels by a few %). Latency-bound kernels (under 2 µs of traffic "
             "at the HBM peak, or no streamed operand) show their achieved rate for reference.", "",
             "| kernel | launches | avg µs | bound | algorithmic work / launch | achieved | of peak | "
             "fetched GB | written GB | traffic / algorithmic bytes | executed MFMA TFLOP/s | MFMA busy | clock GHz |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    gu_row = None
    for name in sorted(KT, key=lambda n: -sum(d for d, _ in KT[n])):
        if name.startswith(("at::native", "__amd")):
            continue
        durs = [d for d, _ in KT[name]]
        avg = sum(durs) / len(durs)
        fb = sum(v for _, v in F.get(name, [])) / max(1, len(F.get(name, []))) * 1024 * ff
        wb = sum(v for _, v in Wr.get(name, [])) / max(1, len(Wr.get(name, []))) * 1024 * fw
        mo = MO.get(name, [])
        mf = sum(v * 512 / d for d, v in mo) / max(1, len(mo)) / 1e12
        gr_all = GR.get(name, [])
        gr = [(d, v) for d, v in gr_all if d >= 200e-6]  # short launches: the counter is not a clock
        clk = sum(v / d for d, v in gr) / len(gr) / 8e9 if gr else None
        mb = MB.get(name, [])
        busy = None
        if mb and len(mb) == len(gr_all) and any(v for _, v in gr_all):
            busy = sum(b for _, b in mb) / (sum(v for _, v in gr_all) / 8.0 * simds)
        base, _, tail = name.partition(" (")
        if base.startswith(SETUP_KERNELS):
            # run once while the bench prepares its inputs, not in the step:
            # its measured traffic rate
            rate = (fb + wb) / avg / 1e9
            lines.append(f"| `{name}` | {len(durs)} | {avg * 1e6:.1f} | setup (not in the step) | - | "
                         f"({rate:.0f} GB/s moved) | ({rate / PEAK_HBM_GBS:.3f}) | {fb / 1e9:.3f} | {wb / 1e9:.3f} "
                         f"| - | 0 | - | {'-' if clk is None else f'{clk:.2f}'} |")
            continue
        key = next((w for w in work if base.startswith(w.partition(" (")[0]) and
                    (not tail or w.endswith("(" + tail))), None)
        bound, amt, unit = work[key] if key else ("latency", None, "")
        if bound == "mfma" and not tail:
            # the FFN GEMMs: HBM-bound below the ridge (decode batches stream weights)
            fb_alg = ffn_bytes[0] if name.endswith("<0>") else ffn_bytes[1]
            if amt / fb_alg < (PEAK_BF16_TFLOPS * 1e12) / (PEAK_HBM_GBS * 1e9):
                bound, amt, unit = "hbm", fb_alg, "B"
        if bound == "hbm" and amt / (PEAK_HBM_GBS * 1e9) < 2e-6:
            bound = "latency"  # under 2 us of traffic at the HBM peak: launch and latency bound
        if bound == "hbm":
            ach, peak, txt = amt / avg / 1e9, PEAK_HBM_GBS, f"{amt / 1e6:.1f} MB"
            alg_bytes = amt
            if name.startswith(("ffn_persistent_kernel", "ffn_skinny_kernel")):
                txt += f" ({(f['ffn_gate_up_flop'] if name.endswith('<0>') else f['ffn_down_flop']) / 1e9:.0f} GFLOP)"
            ach_s = f"{ach:.0f} GB/s"
        elif bound == "mfma":
            ach, peak, txt = amt / avg / 1e12, PEAK_BF16_TFLOPS, f"{amt / 1e12:.3f} TFLOP"
            alg_bytes = ffn_bytes[0] if name.endswith("<0>") else ffn_bytes[1]
            ach_s = f"{ach:.0f} TFLOP/s"
        else:
            ach = peak = None
            alg_bytes = amt if unit == "B" else None
            txt, ach_s = (f"{amt / 1e6:.2f} MB" if alg_bytes else "-"), "-"
            if alg_bytes:
                ach, peak = alg_bytes / avg / 1e9, PEAK_HBM_GBS
                ach_s = f"({ach:.0f} GB/s)"
        frac = f"{ach / peak:.3f}" if ach is not None else "-"
        if bound == "latency" and ach is not None:
            frac = f"({frac})"
        ratio = f"{(fb + wb) / alg_bytes:.2f}" if alg_bytes else "-"
        lines.append(f"| `{name}` | {len(durs)} | {avg * 1e6:.1f} | {bound} | {txt} | {ach_s} | {frac} | "
                     f"{fb / 1e9:.3f} | {wb / 1e9:.3f} | {ratio} | {mf:.0f} | "
                     f"{'-' if not busy else f'{busy:.2f}'} | {'-' if clk is None else f'{clk:.2f}'} |")
        if name == GATE_UP_KERNEL:
            gu_row = (fb, wb)
    lines += ["", "Commands (repository root; each counter set in a run of its own; any output directory):", "",
              "```",
              "export TMPDIR=/tmp; mkdir -p prof",
              "B='python -u bench.py --workload %s --steps 2 --warmup 0 --no-cpu-baseline --no-rank-times "
              "--copy-bytes %d'" % (workload, cb),
              "rocprofv3 --kernel-trace --stats --output-format csv -d prof/kt -o kt -- $B > prof/kt.json",
              "rocprofv3 --pmc FETCH_SIZE --output-format csv -d prof/pmc_f -o p -- $B",
              "rocprofv3 --pmc WRITE_SIZE --output-format csv -d prof/pmc_w -o p -- $B",
              "rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES "
              "GRBM_GUI_ACTIVE --output-format csv -d prof/pmc_m -o p -- $B",
              f"python bench.py --workload {workload} --summarize-profile prof prof/kt.json",
              "```", ""]
    out = os.path.join(ROOT, "profiles", f"kernels_{workload}.md")
    with open(out, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))
    if gu_row is not None:
        tr = {"workload": workload, "kernel": GATE_UP_KERNEL, "kernel_source_sha": _kernel_sha(),
              "ffn_weights": res["config"].get("ffn_weights", "row-major"),
              "fetch_bytes_per_launch": gu_row[0], "write_bytes_per_launch": gu_row[1],
              "fetch_factor": ff, "write_factor": fw, "copy_bytes": cb,
              "bytes_per_launch": gu_row[0] + gu_row[1],
              "note": "FETCH_SIZE and WRITE_SIZE per launch, scaled by copy_bytes / (counter KiB x 1024) "
                      "of a plain device copy of copy_bytes"}
        records = {}
        if os.path.exists(TRAFFIC_JSON):
            with open(TRAFFIC_JSON) as fh:
                records = _traffic_records(json.load(fh))
        records[workload] = tr
        with open(TRAFFIC_JSON, "w") as fh:
            json.dump(records, fh, indent=1)


def _traffic_records(data):
    """The gate/up GEMM's traffic records by workload (a file holding a single
    record is read as one workload's)."""
    return {data["workload"]: data} if "workload" in data else data


STALL_COUNTERS = ["SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_LDS",
                  "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_VMEM",
                  "GRBM_GUI_ACTIVE"]
ISSUE_COUNTERS = ["TA_TA_BUSY", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_VALU", "SQ_INSTS_VMEM",
                  "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE"]


def summarize_counters(workload, prof_dir):
    """Where the waves of the step's long kernels spend their time, from two
    counter runs of the same command (pmc_s: STALL_COUNTERS, pmc_t:
    ISSUE_COUNTERS): shares of wave cycles spent waiting (any dependency; LDS
    results), LDS bank conflicts over LDS-active cycles, and the texture
    unit's busy cycles over the launch's cycles (GRBM_GUI_ACTIVE / 8 XCDs,
    per TA instance, one per CU).  Ratios of counters of one run only, so no
    unit conversion between counter blocks is assumed.  Writes
    profiles/counters_<workload>.md."""
    import collections
    runs = {}
    for sub, names in (("pmc_s", STALL_COUNTERS), ("pmc_t", ISSUE_COUNTERS)):
        path = os.path.join(prof_dir, sub, "p_counter_collection.csv")
        for c in names:
            for i, (n, d, v) in enumerate(_dispatches(path, c)):
                runs.setdefault((sub, n), collections.defaultdict(list))[c].append(v)
    kernels = sorted({n for (_, n) in runs}, key=lambda n: n)
    keep = [n for n in kernels if n.startswith(("gate_topk", "ffn_persistent", "combine_kernel"))]
    lines = [f"# Wave stall counters of the step's long kernels, {workload}, one MI355X", "",
             "Per kernel, averaged over its launches; ratios of counters of one run.  wait any: "
             "SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (waves waiting for any dependency: memory, LDS, barrier); "
             "wait LDS: SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES; LDS conflicts: SQ_LDS_BANK_CONFLICT / "
             "SQ_LDS_IDX_ACTIVE; LDS active: SQ_ACTIVE_INST_LDS / SQ_WAVE_CYCLES; VALU active: "
             "SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES; TA busy: TA_TA_BUSY / (GRBM_GUI_ACTIVE / 8 x CUs); "
             "instruction mix: shares of SQ_INSTS_MFMA, _LDS, _VALU and _VMEM in their sum.", "",
             "| kernel | launches | wait any | wait LDS | LDS active | LDS conflicts | VALU active | TA busy | "
             "MFMA / LDS / VALU / VMEM instructions |",
             "|---|---|---|---|---|---|---|---|---|"]
    cus = 256

    def mean(xs):
        return sum(xs) / len(xs) if xs else float("nan")

    for n in keep:
        s_, t_ = runs.get(("pmc_s", n)), runs.get(("pmc_t", n))
        if not s_ or not t_:
            continue
        wc = s_["SQ_WAVE_CYCLES"]
        r = lambda a, b: mean([x / y for x, y in zip(a, b) if y])  # noqa: E731
        ta = r(t_["TA_TA_BUSY"], [g / 8 * cus for g in t_["GRBM_GUI_ACTIVE"]])
        mix = [mean(t_[c]) for c in ("SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_VALU", "SQ_INSTS_VMEM")]
        tot = sum(mix) or 1.0
        conf = r(s_['SQ_LDS_BANK_CONFLICT'], s_['SQ_LDS_IDX_ACTIVE'])
        lines.append(f"| `{n}` | {len(wc)} | {r(s_['SQ_WAIT_INST_ANY'], wc):.2f} | {r(s_['SQ_WAIT_INST_LDS'], wc):.2f} | "
                     f"{r(s_['SQ_ACTIVE_INST_LDS'], wc):.2f} | "
                     + ("-" if conf != conf else f"{conf:.3f}") + " | "
                     f"{r(s_['SQ_ACTIVE_INST_VALU'], wc):.2f} | {ta:.2f} | "
                     + " / ".join(f"{m / tot:.2f}" for m in mix) + " |")
    cmd = (f"python -u bench.py --workload {workload} --steps 2 --warmup 0 --no-cpu-baseline --no-rank-times")
    lines += ["", "Commands (repository root; each counter set in a run of its own; any output directory):", "",
              "```", "export TMPDIR=/tmp; mkdir -p prof", f"B='{cmd}'",
              "rocprofv3 --pmc " + " ".join(STALL_COUNTERS) + " --output-format csv -d prof/pmc_s -o p -- $B",
              "rocprofv3 --pmc " + " ".join(ISSUE_COUNTERS) + " --output-format csv -d prof/pmc_t -o p -- $B",
              f"python bench.py --workload {workload} --summarize-counters prof", "```", ""]
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", f"counters_{workload}.md")
    with open(out, "w") as fh:
        fh.write("\n".join(lines))
    print("wrote", out)


def summarize_runs(paths, out_name, command):
    """A markdown summary of bench.py result lines (one JSON file each):
    step time, throughput and fractions per workload, the stage medians, the
    balance figures, per-layer or per-step rows, the CPU baseline and any
    side studies.  Written to profiles/<out_name>.md."""
    rows = [json.load(open(p_)) for p_ in paths]
    L = [f"# bench.py results, one MI355X", "", "Command (repository root):", "", "```", command, "```", "",
         "| workload | ms/step (mean / median) | tokens/s | layer MFMA frac | gate/up roofline | FFN MFMA frac "
         "| lookahead hit | spatial static / plan / split | max t_r ms | time-spatial | U_eff |",
         "|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        c, ro, rt, b = r["config"], r["roofline"], r.get("routing", {}), r.get("balance", {})
        L.append(f"| {c['workload']} | {r['ms_per_step']:.4f} / {r.get('ms_per_step_median', 0):.4f} | "
                 f"{r['value']:.0f} | {r['mfma_frac_layer']:.3f} | {ro['frac']:.3f} of {ro['bound']} "
                 f"({ro['achieved']} {ro['unit']}) | {r['ffn_mfma_frac']:.3f} | {rt.get('lookahead_hit', '-')} | "
                 f"{rt.get('spatial_static', '-')} / {rt.get('spatial_plan_even', '-')} / "
                 f"{rt.get('spatial_split', '-')} | {b.get('rank_ffn_max_ms', '-')} | "
                 f"{b.get('time_spatial', '-')} | {b.get('u_eff', '-')} |")
    for r in rows:
        c = r["config"]
        L += ["", f"## {c['workload']}", "", "Stage medians (ms, marked pass): " +
              ", ".join(f"{k} {v}" for k, v in r["stages_ms"].items())]
        if r.get("hbm_frac"):
            L.append("")
            L.append("HBM fractions: " + ", ".join(f"{k} {v}" for k, v in r["hbm_frac"].items()))
        if r.get("units"):
            L += ["", "| unit | ms median | gate/up ms | plan ms (side) | split ms | permute ms | lookahead hit | "
                  "spatial static / plan / split | improved | U_eff |", "|---|---|---|---|---|---|---|---|---|---|"]
            for u in r["units"]:
                st = u["stages_ms"]
                L.append(f"| {u['name']} | {u['ms_median']} | {st['ffn_gate_up_gemm']} | "
                         f"{st['side_histogram_plan']} | {st['split']} | {st['permute']} | {u['lookahead_hit']} | "
                         f"{u['spatial_static']} / {u['spatial_plan_even']} / {u['spatial_split']} | "
                         f"{u['improved']} | {u.get('u_eff', '-')} |")
            L += ["", "Means: " + ", ".join(f"{k} {v}" for k, v in r["units_mean"].items())]
        if r.get("cpu_baseline"):
            cb = r["cpu_baseline"]
            L += ["", f"CPU oracle: {cb['value']:.0f} {cb['unit']} on {cb['cores']} cores ({cb.get('cpu_model')}, "
                  f"BLAS threads {cb.get('blas_threads')}); {cb['sample']}; stage seconds {cb.get('stage_s')}"]
        L += _study_sections(r)
    out = os.path.join(ROOT, "profiles", out_name + ".md")
    with open(out, "w") as fh:
        fh.write("\n".join(L) + "\n")
    print("\n".join(L))


def _study_sections(r):
    """Markdown tables for the side studies of one result line (if present)."""
    L = []
    ts = r.get("two_stage")
    if ts:
        L += ["", "### Two-stage step (MoE_local beside the split and the remote permutation)", "",
              f"Step {ts['ms_per_step']} ms against {r['ms_per_step']:.4f} ms in one stage.", "",
              "| stage | ms |", "|---|---|"]
        L += [f"| {k} | {v} |" for k, v in ts["stages_ms"].items()]
        L += [f"| split stream span: split + remote permutation, waits for free CUs included | {ts['side_work_ms']} |",
              f"| exposed wait on the step's stream | {ts['exposed_ms']} |",
              f"| of the span, overlapping MoE_local | {ts['hidden_ms']} |"]
    sv = r.get("split_variants")
    if sv:
        L += ["", "### Split variants on the step's counts and placement", "",
              "| variant | kernel µs | spatial balance |", "|---|---|---|"]
        L += [f"| {k} | {v['us']} | {v['spatial']} |" for k, v in sv.items()]
    fb = r.get("freebalance")
    if fb:
        L += ["", "### FreeBalance's swaps instead of replicas", "", "| quantity | value |", "|---|---|",
              f"| step ms | {fb['ms_per_step']} |", f"| tokens/s | {fb['tokens_per_s']:.0f} |",
              f"| spatial balance | {fb['spatial']} |", f"| swaps | {fb['swaps']} |",
              f"| planner kernel µs | {fb['plan_us']} |", f"| gamma | {fb['gamma'][0]}/{fb['gamma'][1]} |",
              f"| swap budget per rank | {fb['swaps_per_rank_budget']} |"]
    st = r.get("stale_split")
    if st:
        L += ["", f"### Decision frequency over {st['steps']} step transitions", "",
              "| split | mean spatial balance |", "|---|---|",
              f"| fresh (Relief, every step) | {st['fresh']} |", f"| even | {st['even']} |",
              f"| stale (previous step's shares) | {st['stale']} |", f"| no balancing | {st['static']} |", "",
              f"Stale gives up {st['loss_vs_even']}x the fresh split's gain over the even split; Relief "
              f"{st['relief_us']} µs per call, stale dealing {st['stale_us']} µs."]
    g = r.get("graph")
    if g:
        L += ["", "### The step replayed from a HIP graph", "",
              f"Eager {r['ms_per_step']:.4f} ms, replayed {g['ms_per_step']} ms ({g['tokens_per_s']:.0f} tokens/s)."]
    return L


def _kernel_sha():
    import hashlib
    p = os.path.join(ROOT, "routed_expert_ffn_gate_amd", "csrc", "grouped_ffn.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


if __name__ == "__main__":
    main()
