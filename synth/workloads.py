"""Seeded synthetic workloads shaped like the MoE layers the pages evaluate.

The pages measure on real models and datasets that are not available here
(Libra README, "Running a Single Experiment" and "Requirements": Qwen3-235B-A22B,
GLM-4.5 and eight Hugging Face datasets; the FreeBalance deep dive, section 4:
Qwen3-30B-A3B on LongBench; the Relief summary: routing traces of three MoE
families).  These generators stand in for them with random inputs of the same
shapes:

* hidden states ``h_0 ~ N(0,1)`` and a residual drift ``h_l = h_{l-1} + 0.3 N(0,1)``
  (FreeBalance, eq. 1 and section 3.2: adjacent layers' hidden states are close);
* a linear router ``W ~ N(0, 1/d)`` whose logits are offset by a Zipf-like bias
  ``b_e = -s ln(rank_e)`` over a seeded popularity order (a mixture of two
  popularity orders for the drift workload);
* SwiGLU experts with weights ``~ N(0, 0.02)``.

Every array is drawn as float32 standard normals from
``numpy.random.default_rng(SeedSequence([cid, layer, step, tag, expert]))``,
scaled in float32, and, for bf16 workloads, rounded to bfloat16 with
round-to-nearest-even.  bf16 arrays are returned as raw ``uint16`` bit patterns;
the consumer decides how to widen them.  Nothing here computes any part of the
MoE layer.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace
from typing import Dict, Optional, Tuple

import numpy as np

# Seed tags.
TAG_H0, TAG_DRIFT, TAG_WGATE, TAG_RANK_A, TAG_RANK_B = 1, 2, 3, 4, 5
TAG_W13, TAG_W2, TAG_SHARED_W13, TAG_SHARED_W2 = 6, 7, 8, 9

DRIFT = 0.3          # residual drift scale between consecutive layers
EXPERT_STD = 0.02    # expert (and shared expert) weight std


@dataclass(frozen=True)
class MoEConfig:
    """One workload.  ``L`` is the number of locality imports per rank,
    the whole part of ``N * alpha`` (a rank cannot import half an expert)."""

    name: str
    cid: int
    T: int
    d: int
    E: int
    k: int
    inter: int
    G: int
    N: int
    alpha: float
    L: int
    zipf: float
    dtype: str                  # "f32" or "bf16"
    shared_inter: int = 0       # 0 = no shared expert
    layers: int = 1             # measured layers (drift workload: 8)
    steps: int = 1              # decode steps with re-drawn bias order
    mixture: bool = False       # bias from two popularity orders, weight 0 -> 1

    @property
    def P(self) -> int:
        return self.T * self.k

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


CONFIGS: Dict[str, MoEConfig] = {
    c.name: c
    for c in [
        MoEConfig("c1_tiny_f32", 1, T=256, d=256, E=16, k=2, inter=512, G=4, N=1,
                  alpha=0.5, L=0, zipf=1.2, dtype="f32"),
        MoEConfig("c2_qwen3_30b_decode", 2, T=512, d=2048, E=128, k=8, inter=768, G=8,
                  N=2, alpha=0.5, L=1, zipf=1.2, dtype="bf16", steps=8),
        MoEConfig("c3_qwen3_235b_prefill", 3, T=32768, d=4096, E=128, k=8, inter=1536,
                  G=8, N=4, alpha=0.5, L=2, zipf=1.1, dtype="bf16"),
        MoEConfig("c4_glm45_prefill", 4, T=16384, d=5120, E=160, k=8, inter=1536, G=8,
                  N=4, alpha=0.5, L=2, zipf=1.3, dtype="bf16", shared_inter=1536),
        MoEConfig("c5_olmoe_drift", 5, T=65536, d=2048, E=64, k=8, inter=1024, G=8,
                  N=2, alpha=0.5, L=1, zipf=1.2, dtype="bf16", layers=8, mixture=True),
    ]
}


def config(name: str) -> MoEConfig:
    return CONFIGS[name]


def scaled(cfg: MoEConfig, **changes) -> MoEConfig:
    """A copy of ``cfg`` with some sizes changed (same seed namespace)."""
    return replace(cfg, **changes)


# ---------------------------------------------------------------------------
# primitive draws


def _rng(cfg: MoEConfig, layer: int, step: int, tag: int, expert: int = 0):
    return np.random.default_rng(np.random.SeedSequence([cfg.cid, layer, step, tag, expert]))


def _normal_f32(cfg, shape, layer, step, tag, expert=0) -> np.ndarray:
    return _rng(cfg, layer, step, tag, expert).standard_normal(shape, dtype=np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _as_dtype(cfg: MoEConfig, x_f32: np.ndarray) -> np.ndarray:
    return x_f32.astype(np.float32, copy=False) if cfg.dtype == "f32" else bf16_bits(x_f32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ---------------------------------------------------------------------------
# inputs


def resident_home(cfg: MoEConfig) -> np.ndarray:
    """Resident placement: expert e lives on rank e div (E/G) (contiguous blocks,
    the even expert-device mapping of FreeBalance section 2.2)."""
    return (np.arange(cfg.E, dtype=np.int32) // (cfg.E // cfg.G)).astype(np.int32)


def hidden_states(cfg: MoEConfig, upto: int, step: int = 0) -> list:
    """float32 masters of h_0 .. h_upto (h_0 is the prologue layer's output)."""
    h = _normal_f32(cfg, (cfg.T, cfg.d), 0, step, TAG_H0)
    out = [h]
    for layer in range(1, upto + 1):
        h = (h + np.float32(DRIFT) * _normal_f32(cfg, (cfg.T, cfg.d), layer, step, TAG_DRIFT)).astype(np.float32)
        out.append(h)
    return out


def _popularity_rank(cfg: MoEConfig, layer: int, step: int, tag: int) -> np.ndarray:
    return (1 + _rng(cfg, layer, step, tag).permutation(cfg.E)).astype(np.float64)


def gate_params(cfg: MoEConfig, gate_layer: int, step: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Router of layer ``gate_layer`` (1-based): weight [E,d] in the workload dtype
    (nn.Linear layout) and fp32 bias [E].

    Plain workloads: b_e = -s ln(rank_e), the popularity order drawn per layer and
    (for decode) per step.  Drift workload: two orders A and B drawn once, and
    b_e = ln((1-w) rankA_e^-s + w rankB_e^-s) with w = min((layer-1)/7, 1).
    """
    wstep = 0  # router weights stay fixed across decode steps
    w = _normal_f32(cfg, (cfg.E, cfg.d), gate_layer, wstep, TAG_WGATE) * np.float32(1.0 / math.sqrt(cfg.d))
    s = cfg.zipf
    if cfg.mixture:
        ra = _popularity_rank(cfg, 0, 0, TAG_RANK_A)
        rb = _popularity_rank(cfg, 0, 0, TAG_RANK_B)
        mix = min((gate_layer - 1) / 7.0, 1.0)
        b = np.log((1.0 - mix) * ra ** (-s) + mix * rb ** (-s))
    else:
        r = _popularity_rank(cfg, gate_layer, step, TAG_RANK_A)
        b = -s * np.log(r)
    return _as_dtype(cfg, w.astype(np.float32)), b.astype(np.float32)


def expert_weights(cfg: MoEConfig, layer: int, e: int) -> Tuple[np.ndarray, np.ndarray]:
    """Expert e of measured layer ``layer``: W13 [2*inter, d] (gate rows then up
    rows) and W2 [d, inter], both K-contiguous, in the workload dtype."""
    w13 = _normal_f32(cfg, (2 * cfg.inter, cfg.d), layer, 0, TAG_W13, e)
    w13 *= np.float32(EXPERT_STD)
    w2 = _normal_f32(cfg, (cfg.d, cfg.inter), layer, 0, TAG_W2, e)
    w2 *= np.float32(EXPERT_STD)
    return _as_dtype(cfg, w13), _as_dtype(cfg, w2)


def expert_weights_stacked(cfg: MoEConfig, layer: int) -> Tuple[np.ndarray, np.ndarray]:
    """All experts of one layer stacked: W13 [E,2I,d], W2 [E,d,I]."""
    dt = np.float32 if cfg.dtype == "f32" else np.uint16
    w13 = np.empty((cfg.E, 2 * cfg.inter, cfg.d), dtype=dt)
    w2 = np.empty((cfg.E, cfg.d, cfg.inter), dtype=dt)

    def fill(e):
        a, b = expert_weights(cfg, layer, e)
        w13[e] = a
        w2[e] = b

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(cfg.E)))
    return w13, w2


def shared_weights(cfg: MoEConfig) -> Optional[Tuple[np.ndarray, np.ndarray]]:
    """The always-on shared expert (GLM-4.5 shape): W13 [2*Is, d], W2 [d, Is]."""
    if cfg.shared_inter <= 0:
        return None
    w13 = _normal_f32(cfg, (2 * cfg.shared_inter, cfg.d), 1, 0, TAG_SHARED_W13) * np.float32(EXPERT_STD)
    w2 = _normal_f32(cfg, (cfg.d, cfg.shared_inter), 1, 0, TAG_SHARED_W2) * np.float32(EXPERT_STD)
    return _as_dtype(cfg, w13.astype(np.float32)), _as_dtype(cfg, w2.astype(np.float32))


@dataclass
class LayerInputs:
    """Inputs of one measured layer step.

    ``h_prev`` is the previous layer's output (the prologue's, for the first
    measured layer): the lookahead of the previous step applied gate ``layer``
    to it.  ``h`` is the measured layer's input.  ``w_cur/b_cur`` is the measured
    layer's router, ``w_next/b_next`` the next layer's (the lookahead target).
    """

    cfg: MoEConfig
    layer: int
    step: int
    h_prev: np.ndarray
    h: np.ndarray
    w_cur: np.ndarray
    b_cur: np.ndarray
    w_next: np.ndarray
    b_next: np.ndarray
    home: np.ndarray


def layer_inputs(cfg: MoEConfig, layer: int = 1, step: int = 0, hs: Optional[list] = None) -> LayerInputs:
    """Inputs for measured layer ``layer`` (1-based) at decode step ``step``."""
    if hs is None:
        hs = hidden_states(cfg, layer, step)
    w_cur, b_cur = gate_params(cfg, layer, step)
    w_next, b_next = gate_params(cfg, layer + 1, step)
    return LayerInputs(cfg, layer, step, _as_dtype(cfg, hs[layer - 1]), _as_dtype(cfg, hs[layer]),
                       w_cur, b_cur, w_next, b_next, resident_home(cfg))
