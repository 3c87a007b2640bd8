"""Pins of the oracle's gate, softmax, top-k and lookahead metric (CPU only)."""
import math

import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import workloads as W


def test_widen_bf16_bits_closed_form():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x4049], dtype=np.uint16)
    v = O.widen(bits, "bf16")
    # 1.0, -2.0, 1 + 2^-7, +0, -0, 3.140625
    assert list(v) == [1.0, -2.0, 1.0 + 2.0 ** -7, 0.0, -0.0, 3.140625]


def test_generator_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 3
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 65504.0]  # exact ties
    ours = W.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_router_logits_hand_example():
    # h = [[1, 2], [0.5, -1]], experts' rows W = [[1,0],[0,1],[1,1]], b = [0, .5, -1]
    # z[0] = [1, 2 + .5, 3 - 1] = [1, 2.5, 2];  z[1] = [.5, -1 + .5, -.5 - 1] = [.5, -.5, -1.5]
    h = np.array([[1.0, 2.0], [0.5, -1.0]])
    w = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    b = np.array([0.0, 0.5, -1.0])
    z = O.router_logits(h, w, b)
    assert np.array_equal(z, [[1.0, 2.5, 2.0], [0.5, -0.5, -1.5]])
    idx, gap = O.topk(z, 2)
    assert idx.tolist() == [[1, 2], [0, 1]]
    assert gap.tolist() == [1.0, 1.0]


def test_softmax_closed_forms():
    # equal logits -> 1/E each
    p = O.softmax(np.zeros((1, 5)))
    assert np.allclose(p, 0.2, rtol=0, atol=1e-15)
    # logits differing by ln 3 -> 3/4 and 1/4 (higher logit gets the larger share)
    p = O.softmax(np.array([[math.log(3.0), 0.0]]))
    assert abs(p[0, 0] - 0.75) < 1e-15 and abs(p[0, 1] - 0.25) < 1e-15
    # shift invariance and huge logits (no overflow)
    p = O.softmax(np.array([[1000.0 + math.log(3.0), 1000.0]]))
    assert abs(p[0, 0] - 0.75) < 1e-13


def test_topk_bruteforce_with_ties():
    rng = np.random.default_rng(3)
    for trial in range(50):
        T, E = 7, int(rng.integers(3, 12))
        k = int(rng.integers(1, E + 1))
        z = rng.integers(-3, 4, size=(T, E)).astype(np.float64)  # many exact ties
        idx, gap = O.topk(z, k)
        for t in range(T):
            order = sorted(range(E), key=lambda e: (-z[t, e], e))
            assert idx[t].tolist() == order[:k]
            if k < E:
                assert gap[t] == z[t, order[k - 1]] - z[t, order[k]]
            else:
                assert gap[t] == np.inf


def test_zero_router_weights_pick_highest_bias():
    # W = 0 -> logits are the bias; the selection is the k highest-bias experts,
    # ties to lower id, and the weights are softmax(b) at those experts.
    E, d, k = 6, 8, 3
    b = np.array([0.5, 2.0, -1.0, 2.0, 1.0, 0.0], dtype=np.float32)
    h = np.random.default_rng(0).standard_normal((4, d)).astype(np.float32)
    w0 = np.zeros((E, d), dtype=np.float32)
    idx, w, gap, idx_next, z = O.route(h, w0, b, w0, b, k, "f32")
    assert all(row == [1, 3, 4] for row in idx.tolist())
    assert np.array_equal(idx, idx_next)
    e = np.exp(b.astype(np.float64))
    assert np.allclose(w, (e[[1, 3, 4]] / e.sum())[None, :], rtol=1e-14)
    assert np.allclose(gap, 1.0 - 0.5)


def test_route_weights_are_probabilities():
    cfg = W.scaled(W.config("c1_tiny_f32"), T=64)
    li = W.layer_inputs(cfg)
    idx, w, gap, idx_next, z = O.route(li.h, li.w_cur, li.b_cur, li.w_next, li.b_next, cfg.k, cfg.dtype)
    assert np.all(w > 0) and np.all(w <= 1)
    assert np.all(np.diff(w, axis=1) <= 0)          # listed by descending logit
    assert np.all(gap >= 0)
    p = O.softmax(z)
    assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    for t in range(cfg.T):
        assert len(set(idx[t].tolist())) == cfg.k


def test_lookahead_hit_hand_example_and_identity():
    pred = np.array([[0, 1], [2, 3]])
    act = np.array([[1, 0], [3, 4]])
    assert O.lookahead_hit(pred, act) == 0.75          # (2 + 1) / 4
    # no drift and the same gate -> every assignment is recovered
    cfg = W.scaled(W.config("c1_tiny_f32"), T=64)
    li = W.layer_inputs(cfg)
    i1 = O.route(li.h, li.w_cur, li.b_cur, None, None, cfg.k, cfg.dtype)[0]
    i2 = O.route(li.h, li.w_cur, li.b_cur, None, None, cfg.k, cfg.dtype)[0]
    assert O.lookahead_hit(i1, i2) == 1.0


def test_lookahead_on_drift_is_informative():
    # the drifted hidden state predicts most assignments (a sanity range for
    # these synthetic inputs, not a figure from the pages)
    cfg = W.scaled(W.config("c1_tiny_f32"), T=256)
    li = W.layer_inputs(cfg)
    idx = O.route(li.h, li.w_cur, li.b_cur, None, None, cfg.k, cfg.dtype)[0]
    pred = O.route(li.h_prev, li.w_cur, li.b_cur, None, None, cfg.k, cfg.dtype)[0]
    hit = O.lookahead_hit(pred, idx)
    assert 0.6 < hit < 1.0
