"""Routing-shift metrics on hand-built selections (host only)."""
import numpy as np

from quantized_mixture_experts_qmoe_amd.routing_shift import routing_shift, topk_margin


def test_margin_closed_forms():
    lg = np.array([[3.0, 1.0, 2.0, 0.5], [1.0, 1.0, 1.0, 1.0]])
    assert np.allclose(topk_margin(lg, 1), [1.0, 0.0])
    assert np.allclose(topk_margin(lg, 2), [1.0, 0.0])
    assert np.allclose(topk_margin(lg, 3), [0.5, 0.0])
    assert np.all(np.isinf(topk_margin(lg, 4)))


def test_counts_flips_swaps_and_order():
    # token 0 identical, token 1 one expert replaced, token 2 same set other
    # order, token 3 both experts replaced
    ref = np.array([[0, 1], [2, 3], [1, 0], [0, 1]])
    new = np.array([[0, 1], [2, 4], [0, 1], [2, 3]])
    lg = np.array([[5.0, 4.0, 0.0, 0.0, 0.0],
                   [0.0, 0.0, 5.0, 1.0, 0.9995],    # margin 5e-4
                   [4.0, 5.0, 0.0, 0.0, 0.0],       # margin 4
                   [2.0, 1.95, 1.9, 0.0, 0.0]])     # margin 0.05
    r = routing_shift(ref, new, lg)
    assert r["tokens"] == 4 and r["set_flips"] == 2 and r["experts_swapped"] == 3 and r["order_changes"] == 1
    assert r["flip_rate"] == 0.5
    assert list(r["flipped_tokens"]) == [1, 3]
    # margins: token 0: 4, token 1: 5e-4, token 2: 4, token 3: 0.05
    assert r["margin_hist_all"] == [1, 0, 1, 0, 2]
    assert r["margin_hist_flipped"] == [1, 0, 1, 0, 0]
    assert np.isclose(r["max_flipped_margin"], 0.05)


def test_identical_selections():
    rng = np.random.default_rng(0)
    lg = rng.standard_normal((50, 16))
    idx = np.argsort(-lg, axis=1, kind="stable")[:, :4]
    r = routing_shift(idx, idx.copy(), lg)
    assert r["set_flips"] == 0 and r["experts_swapped"] == 0 and r["order_changes"] == 0
    assert sum(r["margin_hist_all"]) == 50 and r["max_flipped_margin"] == 0.0
