"""Pins of the oracle's SwiGLU experts, weighted combine and the lossless
invariant between the dense MoE definition and the balanced path (CPU only)."""
import math

import numpy as np

from oracle import moe_oracle as O
from synth import workloads as W


def test_silu_closed_forms():
    z = np.array([0.0, math.log(3.0), -math.log(3.0), 40.0, -40.0])
    s = O.silu(z)
    assert s[0] == 0.0
    assert abs(s[1] - 0.75 * math.log(3.0)) < 1e-15          # sigma(ln 3) = 3/4
    assert abs(s[2] + 0.25 * math.log(3.0)) < 1e-15          # sigma(-ln 3) = 1/4
    assert abs(s[3] - 40.0) < 1e-12 and abs(s[4]) < 1e-15


def test_swiglu_hand_example_gate_up_order_and_down_transpose():
    # d = 1, I = 1: W13 = [[ln 3], [2]] (gate row, then up row), W2 = [[0.5]]
    x = np.array([[1.0]])
    w13 = np.array([[math.log(3.0)], [2.0]])
    w2 = np.array([[0.5]])
    y = O.swiglu(x, w13, w2)
    assert abs(y[0, 0] - 0.75 * math.log(3.0) * 2.0 * 0.5) < 1e-15
    # d = 2, I = 1: x = [1, 0]; gate row [ln3, 7], up row [2, 5]; W2 [d=2, I=1] = [[1], [-3]]
    # a = silu(ln 3) * 2 = 1.5 ln 3 ; y = [a * 1, a * -3]
    x = np.array([[1.0, 0.0]])
    w13 = np.array([[math.log(3.0), 7.0], [2.0, 5.0]])
    w2 = np.array([[1.0], [-3.0]])
    y = O.swiglu(x, w13, w2)
    a = 1.5 * math.log(3.0)
    assert np.allclose(y, [[a, -3 * a]], rtol=1e-15, atol=0)


def test_combine_hand_example():
    # T=2, k=2; Y rows: [1,0], [0,1], [2,2], [5,5]; pos = [2, 0, 1, -1]
    Y = np.array([[1.0, 0.0], [0.0, 1.0], [2.0, 2.0], [5.0, 5.0]])
    pos = np.array([2, 0, 1, -1])
    w = np.array([[0.5, 0.25], [0.125, 0.75]])
    out = O.combine(Y, pos, w, 2, 2)
    assert out.tolist() == [[0.5 * 2 + 0.25 * 1, 0.5 * 2], [0.0, 0.125]]
    out2 = O.combine(Y, pos, w, 2, 2, shared=np.ones((2, 2)))
    assert np.array_equal(out2, out + 1)


def _small_layer(seed=0):
    cfg = W.scaled(W.config("c1_tiny_f32"), T=64, d=32, inter=48, E=8, G=4, k=2)
    li = W.layer_inputs(cfg)
    idx, w, gap, idx_next, z = O.route(li.h, li.w_cur, li.b_cur, li.w_next, li.b_next, cfg.k, cfg.dtype)
    experts = {e: tuple(O.widen(a, cfg.dtype) for a in W.expert_weights(cfg, 1, e)) for e in range(cfg.E)}
    return cfg, li, idx, w, experts


def test_lossless_dense_equals_balanced_path():
    cfg, li, idx, w, experts = _small_layer()
    h64 = O.widen(li.h, cfg.dtype)
    c = O.histogram(idx, cfg.G, cfg.E)
    rep = O.plan(c, li.home, cfg.G, cfg.E, cfg.N, cfg.L)
    hc, _ = O.split(c, li.home, rep, cfg.G, cfg.E)
    off, perm, pos = O.permute(idx, li.home, rep, hc, cfg.G, cfg.E)
    dense = O.moe_dense(h64, idx, w, lambda e: experts[e])
    via, _Y = O.moe_via_groups(h64, idx, w, lambda e: experts[e], off, perm, pos, cfg.E)
    assert np.max(np.abs(dense - via)) <= 1e-12 * np.max(np.abs(dense))


def test_single_expert_takes_everything_is_dense_swiglu():
    cfg, li, idx, w, experts = _small_layer()
    h64 = O.widen(li.h, cfg.dtype)
    idx1 = np.full((cfg.T, 1), 3)
    w1 = np.full((cfg.T, 1), 0.5)
    out = O.moe_dense(h64, idx1, w1, lambda e: experts[e])
    ref = 0.5 * O.swiglu(h64, *experts[3])
    assert np.max(np.abs(out - ref)) <= 1e-14 * np.max(np.abs(ref))


def test_moe_dense_token_subset_matches_full():
    cfg, li, idx, w, experts = _small_layer()
    h64 = O.widen(li.h, cfg.dtype)
    full = O.moe_dense(h64, idx, w, lambda e: experts[e])
    toks = np.array([5, 0, 63, 17])
    sub = O.moe_dense(h64, idx, w, lambda e: experts[e], tokens=toks)
    assert np.max(np.abs(sub - full[toks])) <= 1e-12 * np.max(np.abs(full))
