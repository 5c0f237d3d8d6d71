"""Dense routed-expert gated MLP: the output the reader approximates.  (Oracle.)

Channel j of expert e owns row g_j of G_e, row v_j of V_e and column d_j of
D_e; its activation is a_j = phi(g_j^T x) (v_j^T x) and the expert output is
sum_j a_j d_j ([zh §前置知识 / 门控MLP与通道]).  The MoE block output is the
routing-weighted sum over the token's routed experts.  phi is SiLU,
phi(z) = z / (1 + exp(-z)) (reading: the Qwen3 family the pages evaluate).

Pins (tests/test_oracle_reader.py): hand-worked cases with exact BF16 values
(one expert and one channel at H = 2; two weighted experts), which fix the
orientation of D, the activation and the routing weight; the reader's
per-channel decode at k = all channels equals this function on random data.
"""
import numpy as np

from .numerics import weights_f64


def silu(z):
    # exp(-z) overflows to inf for z below about -709, where z / inf = -0 is
    # the right limit: the overflow is expected, not an error
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def dense_moe(gate_bits, up_bits, down_bits, x, ids, w):
    """y = sum_s w_s D_e (phi(G_e x) * (V_e x)), e = ids[s]; float64 [H]."""
    x = np.asarray(x, dtype=np.float64)
    y = np.zeros(x.shape[-1])
    for e, ws in zip(np.asarray(ids).tolist(), np.asarray(w, dtype=np.float64).tolist()):
        g = weights_f64(gate_bits[e]) @ x
        v = weights_f64(up_bits[e]) @ x
        y += ws * (weights_f64(down_bits[e]) @ (silu(g) * v))
    return y
