"""One MoE layer step on one GPU, driven through the libmoelb C ABI.

PyTorch only allocates device memory and supplies the stream; every stage
runs in the HIP library:

  gate_topk (current + lookahead) -> histogram -> split (this step, with the
  plan made one step earlier) -> permute -> grouped SwiGLU FFN (+ shared
  expert) -> combine,
  and, on a side stream after the gate, the lookahead histogram and the plan
  for the next layer, joined before the step ends.  ``step_two_stage`` runs
  the same step with MoE_local (local permutation and FFN over the local
  groups) beside the split and the remote permutation.

The hidden-state rows are read by the gate/up GEMM straight from ``h``
through the permutation (``gather_rows=True``, the default; the permutation
then moves indices only), or from a materialised ``x_perm``
(``gather_rows=False``).  ``materialize_x`` only allocates ``x_perm``.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch

from . import moelb as M

# Stages on the step's stream, in order; the lookahead histogram and the next
# layer's plan run on a side stream (they feed the next step, not this one).
STAGES = ["gate_topk", "histogram", "split", "permute", "grouped_ffn", "combine", "join"]
EVENTS_PER_STEP = 14


def to_device(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Upload an input array unchanged: bf16 bit patterns (uint16) become a
    bfloat16 tensor with the same bits; fp32 stays fp32."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Download a tensor; bfloat16 comes back as uint16 bit patterns."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def pack_expert_weights(w: torch.Tensor, stream=None) -> torch.Tensor:
    """A packed copy of expert weights ([E, rows, K] or one expert's [rows,
    K], bf16) for a layer built with packed_weights=True: done once, when the
    weights are loaded."""
    p = torch.empty_like(w)
    M.moelb_pack_weights(w, p, stream=stream)
    return p


class HipEvents:
    """hipEvent_t handles from libamdhip64, recorded on a stream between
    entry-point calls (the step's stage marks)."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.ev = [ctypes.c_void_p() for _ in range(n)]
        for e in self.ev:
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")

    def record(self, i: int, stream) -> None:
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream if stream is None else stream.cuda_stream)
        if self.hip.hipEventRecord(self.ev[i], s) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        self.hip.hipEventSynchronize(self.ev[b])
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.ev[a], self.ev[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


@dataclass
class StepOut:
    idx: torch.Tensor
    wts: torch.Tensor
    gap: torch.Tensor
    idx_next: torch.Tensor
    counts: torch.Tensor
    counts_next: torch.Tensor
    replica_next: torch.Tensor
    plan_load_next: torch.Tensor
    host_count: torch.Tensor
    load: torch.Tensor
    group_off: torch.Tensor
    perm: torch.Tensor
    pos: torch.Tensor
    x_perm: Optional[torch.Tensor]
    y: torch.Tensor
    shared: Optional[torch.Tensor]
    out: torch.Tensor
    home_next: Optional[torch.Tensor] = None  # FreeBalance: the next layer's placement


class MoELayer:
    """Device buffers and the stage sequence of one layer step.

    Shapes: T tokens, d hidden, E experts, top-k, inter, G virtual ranks, N
    replica slots, L locality imports; ``dtype`` "bf16" or "f32"."""

    def __init__(self, T, d, E, k, inter, G, N, L, dtype, device="cuda", shared_inter=0, passes=12,
                 gather_rows=True, materialize_x=False, balancer="libra", fb_tau=0, fb_gamma=None,
                 fb_budget=None, packed_weights=False, overlap_split=None):
        """balancer "libra": replication plan (N slots, L locality imports)
        and the per-step split; "freebalance": expert swaps instead (no
        replicas; at most fb_budget swaps per rank, default N; threshold
        fb_tau; gamma = fb_gamma (num, den), default 1 / the mean rank load).
        packed_weights: the expert (and shared) weights passed to the steps
        are in moelb_pack_weights' layout.  overlap_split: run the split
        beside the local half of the permutation (default: wherever the
        permutation is not a single launch anyway, i.e. more than 8192 pairs,
        E*G > 2048 or rows copied)."""
        self.T, self.d, self.E, self.k, self.inter = T, d, E, k, inter
        self.ffn_opt = M.MOELB_FFN_PACKED_WEIGHTS if packed_weights else 0
        self.G, self.N, self.L, self.passes = G, N, L, passes
        if balancer not in ("libra", "freebalance"):
            raise ValueError(balancer)
        self.balancer = balancer
        self.fb_tau = fb_tau
        self.fb_gamma = fb_gamma if fb_gamma is not None else (1, min(1 << 20, max(1, (T * k) // G)))
        self.fb_budget = fb_budget if fb_budget is not None else N
        self.dtype = dtype
        self.tdtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.dev = torch.device(device)
        self.gather_rows = gather_rows
        self.materialize_x = materialize_x or not gather_rows
        P = T * k
        i32 = dict(dtype=torch.int32, device=self.dev)
        self.P = P
        self.idx = torch.empty((T, k), **i32)
        self.idx_next = torch.empty((T, k), **i32)
        self.wts = torch.empty((T, k), dtype=torch.float32, device=self.dev)
        self.gap = torch.empty((T,), dtype=torch.float32, device=self.dev)
        self.counts = torch.empty((G, E), **i32)
        self.counts_next = torch.empty((G, E), **i32)
        self.replica_next = torch.empty((G, N), **i32)
        self.plan_load_next = torch.empty((G,), **i32)
        self.host_count = torch.empty((E, G), **i32)
        self.load = torch.empty((G,), **i32)
        self.group_off = torch.empty((2 * G * E + 1,), **i32)
        self.perm = torch.empty((P,), **i32)
        self.pos = torch.empty((P,), **i32)
        self.x_perm = torch.empty((P, d), dtype=self.tdtype, device=self.dev) if self.materialize_x else None
        self.y = torch.empty((P, d), dtype=self.tdtype, device=self.dev)
        self.out = torch.empty((T, d), dtype=self.tdtype, device=self.dev)
        self.shared_inter = shared_inter
        self.shared = torch.empty((T, d), dtype=self.tdtype, device=self.dev) if shared_inter > 0 else None
        self.shared_off = torch.tensor([0, T], **i32) if shared_inter > 0 else None
        code = M.MOELB_BF16 if dtype == "bf16" else M.MOELB_F32
        self.ws_perm = torch.empty((max(1, M.moelb_permute_workspace_bytes(T, k, E, G)),), dtype=torch.uint8,
                                   device=self.dev)
        self.ws_ffn = torch.empty((max(1, M.moelb_grouped_ffn_workspace_bytes(P, 2 * G * E, E, d, inter, code)),),
                                  dtype=torch.uint8, device=self.dev)
        self.side = torch.cuda.Stream(device=self.dev)  # default priority
        self.ev_gate = torch.cuda.Event()
        self.ev_side = torch.cuda.Event()
        # two-stage schedule: split and remote permutation beside MoE_local
        self.side2 = torch.cuda.Stream(device=self.dev)  # default priority
        self.ev_hist = torch.cuda.Event()
        self.ev_local = torch.cuda.Event()
        self.ev_remote = torch.cuda.Event()
        self.ev_split = torch.cuda.Event()
        if overlap_split is None:
            overlap_split = (not gather_rows) or T * k > 8192 or E * G > 2048
        self.overlap_split = overlap_split
        # round schedules of the split, made once per placement (Relief): for
        # the placement in force and for the next layer's
        self.sched_cur = torch.full((M.MOELB_SPLIT_SCHEDULE_INTS,), -1, **i32)
        self.sched_next = torch.full((M.MOELB_SPLIT_SCHEDULE_INTS,), -1, **i32)
        # advance(): the next layer's plan becomes the one in force while the
        # next step writes its own next plan into the other buffer
        self.replica_spare = torch.empty((G, N), **i32)
        if balancer == "freebalance":
            self.home_next = torch.empty((E,), **i32)
            self.swaps_next = torch.empty((E // 2 + 1, 2), **i32)
            self.n_swaps_next = torch.empty((1,), **i32)
            self.home_base = None
        self.ws_shared = None
        if shared_inter > 0:
            self.ws_shared = torch.empty((M.moelb_grouped_ffn_workspace_bytes(T, 1, 1, d, shared_inter, code),),
                                         dtype=torch.uint8, device=self.dev)

    # -- stages ---------------------------------------------------------------

    def predict_plan(self, h_prev, w_cur, b_cur, home, replica_out, stream=None):
        """Prologue: the previous step's lookahead for this layer (gate of this
        layer on the previous hidden states), its histogram and plan."""
        M.moelb_gate_topk(h_prev, w_cur, b_cur, None, None, self.idx_next, self.wts, None, None, stream=stream)
        M.moelb_histogram(self.idx_next, self.G, self.counts_next, stream=stream)
        M.moelb_plan(self.counts_next, home, self.L, replica_out, None, stream=stream)
        M.moelb_split_schedule(home, replica_out, self.sched_cur, self.G, stream=stream)

    def predict_placement(self, h_prev, w_cur, b_cur, home_base, home_out, stream=None):
        """FreeBalance prologue: the early router (this layer's gate on the
        previous hidden states), its histogram, and the swaps from the base
        placement ``home_base`` (kept as the next layer's starting placement)
        into ``home_out``."""
        M.moelb_gate_topk(h_prev, w_cur, b_cur, None, None, self.idx_next, self.wts, None, None, stream=stream)
        M.moelb_histogram(self.idx_next, self.G, self.counts_next, stream=stream)
        self.home_base = home_base
        self._plan_swaps(home_out, stream)

    def _plan_swaps(self, home_out, stream):
        M.moelb_plan_swaps(self.counts_next, self.home_base, home_out, self.plan_load_next, tau=self.fb_tau,
                           gamma=self.fb_gamma, max_swaps_per_rank=self.fb_budget, swaps=self.swaps_next,
                           n_swaps=self.n_swaps_next, stream=stream)

    def _plan_next(self, home):
        """The next layer's balancing, on the side stream."""
        if self.balancer == "freebalance":
            self._plan_swaps(self.home_next, self.side)
        else:
            M.moelb_plan(self.counts_next, home, self.L, self.replica_next, self.plan_load_next, stream=self.side)
            M.moelb_split_schedule(home, self.replica_next, self.sched_next, self.G, stream=self.side)

    def advance(self) -> torch.Tensor:
        """Make the plan this step made for the next layer the one in force
        (Libra "Key Ideas": the lookahead plan of layer i+1 is applied at
        layer i+1): returns its replica table, to pass as ``replica_cur`` to
        the next step, and the split schedule made beside it becomes the one
        the split reads.  The buffers are swapped, not copied, so the next
        step's own plan does not overwrite the placement in force."""
        self.replica_next, self.replica_spare = self.replica_spare, self.replica_next
        self.sched_cur, self.sched_next = self.sched_next, self.sched_cur
        return self.replica_spare

    def _ffn(self, h, w13, w2, mark=None, stream=None):
        """The grouped FFN over every group; with ``mark``, its three stages
        are launched apart and marks 8..11 recorded around them."""
        x = h if self.gather_rows else self.x_perm
        kw = dict(G=self.G, stream=stream)
        if self.gather_rows:
            kw.update(gather=self.perm, gather_k=self.k)
        if mark is None:
            M.moelb_grouped_ffn_stages(M.MOELB_FFN_ALL | self.ffn_opt, x, self.P, self.group_off, self.E, w13, w2,
                                       self.ws_ffn, self.y, **kw)
            return
        for i, stage in enumerate((M.MOELB_FFN_SCHEDULE, M.MOELB_FFN_GATE_UP, M.MOELB_FFN_DOWN)):
            mark(8 + i)
            M.moelb_grouped_ffn_stages(stage | self.ffn_opt, x, self.P, self.group_off, self.E, w13, w2,
                                       self.ws_ffn, self.y, **kw)
        mark(11)

    def _shared_ffn(self, h, shared_w13, shared_w2, stream):
        M.moelb_grouped_ffn_stages(M.MOELB_FFN_ALL | self.ffn_opt, h, self.T, self.shared_off, 1, shared_w13,
                                   shared_w2, self.ws_shared, self.shared, stream=stream)

    def _out(self):
        return StepOut(self.idx, self.wts, self.gap, self.idx_next, self.counts, self.counts_next, self.replica_next,
                       self.plan_load_next, self.host_count, self.load, self.group_off, self.perm, self.pos,
                       self.x_perm, self.y, self.shared, self.out,
                       self.home_next if self.balancer == "freebalance" else None)

    def step(self, h, w_cur, b_cur, w_next, b_next, home, replica_cur, w13, w2, shared_w13=None, shared_w2=None,
             stream=None, events: Optional[HipEvents] = None, ev_base: int = 0, sched=None) -> StepOut:
        """One layer step.  With ``events``, marks ev_base+0..7 bracket the
        stages of STAGES on the step's stream, ev_base+8..11 bracket the
        grouped FFN's three stages (schedule, gate/up GEMM, down GEMM, each
        launched on its own), ev_base+12..13 bracket the side stream's work.
        ``sched``: the split's round schedule for ``replica_cur`` (default: the
        one ``predict_plan`` or ``advance`` left in force)."""
        ev = events
        s0 = stream if stream is not None else torch.cuda.current_stream()

        def mark(i, st=None):
            if ev is not None:
                ev.record(ev_base + i, st if st is not None else s0)

        mark(0)
        M.moelb_gate_topk(h, w_cur, b_cur, w_next, b_next, self.idx, self.wts, self.gap, self.idx_next, stream=s0)
        self.ev_gate.record(s0)
        # side stream: lookahead histogram and the next layer's plan
        self.side.wait_event(self.ev_gate)
        mark(12, self.side)
        M.moelb_histogram(self.idx_next, self.G, self.counts_next, stream=self.side)
        self._plan_next(home)
        mark(13, self.side)
        self.ev_side.record(self.side)
        mark(1)
        M.moelb_histogram(self.idx, self.G, self.counts, stream=s0)
        mark(2)
        sched_ = self.sched_cur if sched is None else sched
        copy_rows = not self.gather_rows  # the gather GEMM reads h through perm instead
        hr, xr = (h, self.x_perm) if copy_rows else (None, None)
        code = M.MOELB_BF16 if self.dtype == "bf16" else M.MOELB_F32
        if self.overlap_split:
            # the split beside the local half of the permutation (local groups
            # and their order do not depend on it: Libra "Key Ideas", MoE_local
            # needs no sharding decision), the remote half after both; the
            # outputs are moelb_permute's.  Mark 3 closes the split on its
            # stream, so "permute" is what the permutation leaves after it.
            self.ev_hist.record(s0)
            self.side2.wait_event(self.ev_hist)
            M.moelb_split_scheduled(self.counts, home, replica_cur, sched_, self.host_count, self.load,
                                    passes=self.passes, stream=self.side2)
            mark(3, self.side2)
            self.ev_split.record(self.side2)
            M.moelb_permute_local(hr, self.idx, self.G, home, replica_cur, self.ws_perm, self.group_off, self.perm,
                                  self.pos, xr, d=self.d, dtype=code, stream=s0)
            s0.wait_event(self.ev_split)
            M.moelb_permute_remote(hr, self.idx, self.G, home, replica_cur, self.host_count, self.ws_perm,
                                   self.group_off, self.perm, self.pos, xr, d=self.d, dtype=code, stream=s0)
        else:
            M.moelb_split_scheduled(self.counts, home, replica_cur, sched_, self.host_count, self.load,
                                    passes=self.passes, stream=s0)
            mark(3)
            M.moelb_permute(hr, self.idx, self.G, home, replica_cur, self.host_count, self.ws_perm, self.group_off,
                            self.perm, self.pos, xr, d=self.d, dtype=code, stream=s0)
        mark(4)
        self._ffn(h, w13, w2, mark if ev is not None else None, stream=s0)
        if self.shared is not None:
            self._shared_ffn(h, shared_w13, shared_w2, s0)
        mark(5)
        M.moelb_combine(self.y, self.pos, self.wts, self.out, shared=self.shared, stream=s0)
        mark(6)
        s0.wait_event(self.ev_side)
        mark(7)
        return self._out()


    def step_two_stage(self, h, w_cur, b_cur, w_next, b_next, home, replica_cur, w13, w2, shared_w13=None,
                       shared_w2=None, stream=None, events: Optional[HipEvents] = None, ev_base: int = 0) -> StepOut:
        """The same layer step in two stages (Libra README "Key Ideas":
        MoE_local starts right after gating, the token sharding runs beside
        it).  After the histogram, the step's stream places the local pairs
        and runs the grouped FFN over the local groups while a second stream
        runs the split and places the remote pairs; the remote groups follow.
        Outputs are identical to ``step``'s.  Event marks (TWO_STAGE_MARKS):
        ev_base+0..8 on the step's stream, +9..11 on the split stream, +12..13
        on the lookahead stream."""
        ev = events
        s0 = stream if stream is not None else torch.cuda.current_stream()
        GE = self.G * self.E
        code = M.MOELB_BF16 if self.dtype == "bf16" else M.MOELB_F32
        copy_rows = not self.gather_rows

        def mark(i, st=None):
            if ev is not None:
                ev.record(ev_base + i, st if st is not None else s0)

        def ffn(off):
            all_ = M.MOELB_FFN_ALL | self.ffn_opt
            if self.gather_rows:
                M.moelb_grouped_ffn_stages(all_, h, self.P, off, self.E, w13, w2, self.ws_ffn, self.y, G=self.G,
                                           gather=self.perm, gather_k=self.k, stream=s0)
            else:
                M.moelb_grouped_ffn_stages(all_, self.x_perm, self.P, off, self.E, w13, w2, self.ws_ffn, self.y,
                                           G=self.G, stream=s0)

        mark(0)
        M.moelb_gate_topk(h, w_cur, b_cur, w_next, b_next, self.idx, self.wts, self.gap, self.idx_next, stream=s0)
        self.ev_gate.record(s0)
        self.side.wait_event(self.ev_gate)
        mark(12, self.side)
        M.moelb_histogram(self.idx_next, self.G, self.counts_next, stream=self.side)
        self._plan_next(home)
        mark(13, self.side)
        self.ev_side.record(self.side)
        mark(1)
        M.moelb_histogram(self.idx, self.G, self.counts, stream=s0)
        self.ev_hist.record(s0)
        mark(2)
        # split stream: the split needs only the counts
        self.side2.wait_event(self.ev_hist)
        mark(9, self.side2)
        M.moelb_split_scheduled(self.counts, home, replica_cur, self.sched_cur, self.host_count, self.load,
                                passes=self.passes, stream=self.side2)
        mark(10, self.side2)
        M.moelb_permute_local(h if copy_rows else None, self.idx, self.G, home, replica_cur, self.ws_perm,
                              self.group_off, self.perm, self.pos, self.x_perm if copy_rows else None, d=self.d,
                              dtype=code, stream=s0)
        self.ev_local.record(s0)
        mark(3)
        self.side2.wait_event(self.ev_local)
        M.moelb_permute_remote(h if copy_rows else None, self.idx, self.G, home, replica_cur, self.host_count,
                               self.ws_perm, self.group_off, self.perm, self.pos, self.x_perm if copy_rows else None,
                               d=self.d, dtype=code, stream=self.side2)
        mark(11, self.side2)
        self.ev_remote.record(self.side2)
        ffn(self.group_off[:GE + 1])  # MoE_local
        mark(4)
        s0.wait_event(self.ev_remote)
        mark(5)
        ffn(self.group_off[GE:])  # MoE_remote
        if self.shared is not None:
            self._shared_ffn(h, shared_w13, shared_w2, s0)
        mark(6)
        M.moelb_combine(self.y, self.pos, self.wts, self.out, shared=self.shared, stream=s0)
        mark(7)
        s0.wait_event(self.ev_side)
        mark(8)
        return self._out()


# Event marks of step_two_stage: (name, first, last) -> elapsed between them.
TWO_STAGE_MARKS = {
    "gate_topk": (0, 1), "histogram": (1, 2), "permute_local": (2, 3), "ffn_local": (3, 4),
    "wait_remote": (4, 5), "ffn_remote": (5, 6), "combine": (6, 7), "join": (7, 8),
    "split": (9, 10), "permute_remote": (10, 11), "side_histogram_plan": (12, 13),
}


def stage_times_ms(ev: HipEvents, base: int = 0) -> Dict[str, float]:
    """Per-stage times of a step recorded with ``events`` at ``base``."""
    t = {name: ev.elapsed_ms(base + i, base + i + 1) for i, name in enumerate(STAGES)}
    t["ffn_schedule"] = ev.elapsed_ms(base + 8, base + 9)
    t["ffn_gate_up_gemm"] = ev.elapsed_ms(base + 9, base + 10)
    t["ffn_down_gemm"] = ev.elapsed_ms(base + 10, base + 11)
    t["side_histogram_plan"] = ev.elapsed_ms(base + 12, base + 13)
    return t
