"""Softmax top-k router of the MoE layer.  (Oracle: test infrastructure.)

The router activates a few experts per token, e.g. 8 of 128
([zh §前置知识 / Mixture-of-Experts (MoE)]); the routing weight w_j of a
channel is the weight of its expert ([zh §核心方法]).

Reading (Qwen3 convention): logits = W_router x, probabilities = softmax over
all experts, keep the ``top`` largest (ties -> lower expert index), then
renormalise the kept probabilities to sum to one.  The router decision is an
argmax taken on floating point, so tests compare the library's choice with
this one outside a relative tie band.

Pins (tests/test_oracle_route.py): brute-force ordering, renormalisation
invariance of the reader's kept set.
"""
import numpy as np

from .numerics import bf16_to_f64


def route(router_bits, x, top):
    """Returns (ids int32 [top] sorted by weight desc, weights float64 [top], logits)."""
    logits = bf16_to_f64(router_bits) @ np.asarray(x, dtype=np.float64)
    m = logits.max()
    p = np.exp(logits - m)
    p = p / p.sum()
    order = np.lexsort((np.arange(p.shape[0]), -p))[:top]
    w = p[order] / p[order].sum()
    return order.astype(np.int32), w, logits
