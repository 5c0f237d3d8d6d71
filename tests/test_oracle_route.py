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
