"""Pins for the softmax top-k router."""
import numpy as np

from oracle.route import route
from synth import f32_to_bf16_bits


def test_route_brute_force():
    rng = np.random.default_rng(3)
    router = f32_to_bf16_bits(rng.standard_normal((16, 32)).astype(np.float32) * 0.3)
    for _ in range(50):
        x = rng.standard_normal(32).astype(np.float32)
        ids, w, logits = route(router, x, 4)
        order = sorted(range(16), key=lambda e: (-logits[e], e))[:4]
        assert ids.tolist() == order
        assert abs(w.sum() - 1.0) < 1e-12 and np.all(np.diff(w) <= 0)
        p = np.exp(logits - logits.max())
        p /= p.sum()
        assert np.allclose(w, p[order] / p[order].sum())


def test_route_ties_go_to_the_lower_index():
    # rows repeated in pairs: each logit ties exactly with its twin's
    rng = np.random.default_rng(4)
    base = f32_to_bf16_bits(rng.standard_normal((4, 32)).astype(np.float32) * 0.3)
    router = np.repeat(base, 2, axis=0)  # experts 2i and 2i + 1 share a row
    x = rng.standard_normal(32).astype(np.float32)
    ids, w, logits = route(router, x, 4)
    assert logits[0::2].tolist() == logits[1::2].tolist()
    assert ids[0] % 2 == 0 and ids[1] == ids[0] + 1 and ids[2] % 2 == 0 and ids[3] == ids[2] + 1
    assert w[0] == w[1] and w[2] == w[3]


def test_route_two_experts_closed_form():
    # bf16-exact rows and token: logits are exact small integers, and the
    # renormalised weights of two experts are the logistic of their gap
    router = f32_to_bf16_bits(np.array([[1.0, 2.0, 0.0, -1.0], [0.5, 0.0, 1.0, 0.0]], np.float32))
    x = np.array([1.0, 1.0, 2.0, 1.0], np.float32)  # logits 2.0 and 2.5
    ids, w, logits = route(router, x, 2)
    assert logits.tolist() == [2.0, 2.5]
    assert ids.tolist() == [1, 0]
    s = 1.0 / (1.0 + np.exp(-0.5))
    assert abs(w[0] - s) < 1e-15 and abs(w[1] - (1.0 - s)) < 1e-15
    ids1, w1, _ = route(router, x, 1)
    assert ids1.tolist() == [1] and w1.tolist() == [1.0]
