"""Seeded synthetic workloads for the channel-selection reader.

This module only draws random numbers and lays them out.  It holds none of
the reader's arithmetic (no rotation, no sketch, no scoring, no routing), so
both the CPU oracle and the HIP library may consume what it produces.

Shapes follow the MoE layers the channel-selection pages evaluate: the
Qwen3-30B-A3B layer (hidden 2048, 128 experts, expert intermediate 768, 8
routed experts, i.e. 6144 candidate channels per token) and the
Qwen3-235B-A22B layer (hidden 4096, 128 experts, intermediate 1536), plus a
tiny layer for fast checks.  The model table of the expert-prefetching page
("Speculating Experts Accelerates MoE Inference", section 实验设置) gives the
same layer shapes.

Value recipe (no trained weights exist here):
  * gate, up, down and router weights ~ N(0, 0.02) drawn in float32, then
    rounded to bfloat16 (round to nearest even);
  * a seeded set of "outlier" hidden coordinates: the gate and up columns at
    those coordinates are multiplied by ``w_outlier_mult`` before rounding;
  * tokens x ~ N(0, 1) in float32, with ``x_outlier_dims`` seeded hidden
    dimensions multiplied by ``x_outlier_mult`` (the same dimensions for
    every token of a workload).

Every array comes from its own numpy ``default_rng([seed, stream, ...])``
streams, so one array can be regenerated without the others.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

__all__ = [
    "LayerShape", "Workload", "WORKLOADS", "workload", "f32_to_bf16_bits",
    "bf16_bits_to_f32", "make_layer", "make_layer_q4", "q4_row_bytes", "make_tokens",
    "make_routing_inputs",
]


@dataclass(frozen=True)
class LayerShape:
    hidden: int          # H
    n_experts: int       # E
    inter: int           # I, expert intermediate size (channels per expert)
    top: int             # routed experts per token
    rank: int = 32       # recovery rank
    n_screen: int = 80   # coordinates screened per 128-block
    block: int = 128     # rotation block

    @property
    def n_blocks(self) -> int:
        return self.hidden // self.block

    @property
    def n_cand(self) -> int:
        return self.top * self.inter


@dataclass(frozen=True)
class Workload:
    name: str
    shape: LayerShape
    batch: int
    ks: tuple            # top-k budgets exercised on this workload
    weight_seed: int
    token_seed: int
    n_tokens: int
    n_layers: int = 1
    w_std: float = 0.02
    w_outlier_frac: float = 0.005
    w_outlier_mult: float = 20.0
    x_outlier_dims: int = 4
    x_outlier_mult: float = 30.0
    rot_seed: int = 0x5EED_0000_CAFE_F00D
    notes: str = ""
    extra: dict = field(default_factory=dict)

    def n_w_outliers(self) -> int:
        return int(round(self.w_outlier_frac * self.shape.hidden))


_QWEN3_30B = LayerShape(hidden=2048, n_experts=128, inter=768, top=8)
_QWEN3_235B = LayerShape(hidden=4096, n_experts=128, inter=1536, top=8)
_TINY = LayerShape(hidden=256, n_experts=16, inter=64, top=2)

WORKLOADS = {
    # 128 candidates; k = 18% of them.
    "tiny": Workload("tiny", _TINY, batch=1, ks=(23,), weight_seed=0,
                     token_seed=100, n_tokens=64, w_outlier_frac=0.01,
                     x_outlier_dims=0, x_outlier_mult=1.0),
    # k = 756 is about 17.8% of the dense routed-expert bytes, k = 445 about 12.8%.
    "qwen3-30b-a3b": Workload("qwen3-30b-a3b", _QWEN3_30B, batch=1, ks=(756, 445),
                              weight_seed=0, token_seed=1, n_tokens=256),
    "qwen3-30b-a3b-b4": Workload("qwen3-30b-a3b-b4", _QWEN3_30B, batch=4, ks=(445, 756),
                                 weight_seed=0, token_seed=4, n_tokens=256),
    "qwen3-30b-a3b-48l": Workload("qwen3-30b-a3b-48l", _QWEN3_30B, batch=1, ks=(756,),
                                  weight_seed=1000, token_seed=2, n_tokens=512,
                                  n_layers=48),
    # k = 12.3% of 12288 candidates.
    "qwen3-235b-a22b": Workload("qwen3-235b-a22b", _QWEN3_235B, batch=8, ks=(1511,),
                                weight_seed=3, token_seed=5, n_tokens=256),
}


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


# --- bfloat16 bit handling (input generation only) ------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, nearest-even; returns uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --- generators ------------------------------------------------------------

_STREAM_GATE, _STREAM_UP, _STREAM_DOWN, _STREAM_ROUTER, _STREAM_WOUT = 1, 2, 3, 4, 5
_STREAM_TOK, _STREAM_XOUT, _STREAM_IDS, _STREAM_GW = 11, 12, 13, 14


def _rng(seed: int, stream: int, sub: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream), int(sub)])


def weight_outlier_coords(wl: Workload, layer: int = 0) -> np.ndarray:
    n = wl.n_w_outliers()
    rng = _rng(wl.weight_seed + layer, _STREAM_WOUT)
    return np.sort(rng.choice(wl.shape.hidden, size=n, replace=False)).astype(np.int64)


def x_outlier_dims(wl: Workload) -> np.ndarray:
    rng = _rng(wl.token_seed, _STREAM_XOUT)
    return np.sort(rng.choice(wl.shape.hidden, size=wl.x_outlier_dims, replace=False)).astype(np.int64)


_CHUNK_ROWS = 4096


def _pool_size() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except (AttributeError, OSError):
        return max(1, min(16, os.cpu_count() or 1))


def _normal_bf16(seed, stream, shape, std, col_scale=None):
    """N(0, std) float32 rounded to bf16.

    ``shape`` is (..., H); ``col_scale`` multiplies the last axis before
    rounding.  Rows come in chunks of 4096, chunk c from its own stream
    ``default_rng([seed, stream, 1 + c])``, so the result does not depend on
    how many threads fill it (numpy's generators release the GIL while they
    fill an array).
    """
    rows = int(np.prod(shape[:-1]))
    cols = shape[-1]
    out = np.empty((rows, cols), dtype=np.uint16)

    def fill(c):
        r0 = c * _CHUNK_ROWS
        r1 = min(rows, r0 + _CHUNK_ROWS)
        a = _rng(seed, stream, 1 + c).standard_normal((r1 - r0, cols), dtype=np.float32)
        a *= np.float32(std)
        if col_scale is not None:
            a *= col_scale
        out[r0:r1] = f32_to_bf16_bits(a)

    n = -(-rows // _CHUNK_ROWS)
    if n == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_pool_size()) as ex:
            list(ex.map(fill, range(n)))
    return out.reshape(shape)


def make_layer(wl: Workload, layer: int = 0) -> dict:
    """Weights of one routed-expert layer as bf16 bit patterns (uint16).

    gate, up: [E][I][H]   (row j of G_e / V_e is channel j's input weights)
    down:     [E][H][I]   (column j of D_e is channel j's output direction)
    router:   [E][H]
    """
    s = wl.shape
    seed = wl.weight_seed + layer
    col = np.ones(s.hidden, dtype=np.float32)
    col[weight_outlier_coords(wl, layer)] = np.float32(wl.w_outlier_mult)
    gate = _normal_bf16(seed, _STREAM_GATE, (s.n_experts, s.inter, s.hidden), wl.w_std, col)
    up = _normal_bf16(seed, _STREAM_UP, (s.n_experts, s.inter, s.hidden), wl.w_std, col)
    down = _normal_bf16(seed, _STREAM_DOWN, (s.n_experts, s.hidden, s.inter), wl.w_std)
    router = _normal_bf16(seed, _STREAM_ROUTER, (s.n_experts, s.hidden), wl.w_std)
    return {"gate": gate, "up": up, "down": down, "router": router}


def q4_row_bytes(hidden: int) -> int:
    """Bytes of one 4-bit row record of `hidden` weights (see make_layer_q4)."""
    return -(-(hidden // 2 + 3 * (hidden // 128)) // 16) * 16


def _quantize_rows_q4(rows: np.ndarray, group: int = 128) -> np.ndarray:
    """Round-to-nearest asymmetric 4-bit quantisation of float32 rows [n][H],
    one fp16 scale and one zero point per group of 128: scale = (max - min)
    / 15 rounded to fp16 (1 when a group is constant), zero = round(-min /
    scale) clamped to 0..15, q = round(w / scale) + zero clamped to 0..15.
    Returns the row records [n][q4_row_bytes(H)] (codes two per byte, even
    index in the low nibble; then the fp16 scales; then the zero points)."""
    n, H = rows.shape
    g = rows.reshape(n, H // group, group).astype(np.float32)
    mn, mx = g.min(axis=2), g.max(axis=2)
    scale = ((mx - mn) / np.float32(15)).astype(np.float16)
    scale[scale == 0] = np.float16(1)
    sc = scale.astype(np.float32)
    zero = np.clip(np.rint(-mn / sc), 0, 15).astype(np.uint8)
    q = np.clip(np.rint(g / sc[..., None]) + zero[..., None], 0, 15).astype(np.uint8).reshape(n, H)
    rec = np.zeros((n, q4_row_bytes(H)), dtype=np.uint8)
    rec[:, :H // 2] = q[:, 0::2] | (q[:, 1::2] << 4)
    rec[:, H // 2:H // 2 + 2 * (H // group)] = scale.view(np.uint8).reshape(n, -1)
    rec[:, H // 2 + 2 * (H // group):H // 2 + 3 * (H // group)] = zero
    return rec


def make_layer_q4(wl: Workload, layer: int = 0) -> dict:
    """A synthetic 4-bit (GPTQ-like storage) checkpoint of the layer
    make_layer draws: every channel's gate row, up row and down column
    (over the hidden units) quantised per group of 128 hidden units
    (_quantize_rows_q4).  Returns {"rows": uint8 [E][I][3][q4_row_bytes(H)]
    (gate, up, down record of each channel), "router": bf16 [E][H]}."""
    L = make_layer(wl, layer)
    s = wl.shape
    rows = np.empty((s.n_experts, s.inter, 3, q4_row_bytes(s.hidden)), dtype=np.uint8)
    for e in range(s.n_experts):
        rows[e, :, 0] = _quantize_rows_q4(bf16_bits_to_f32(L["gate"][e]))
        rows[e, :, 1] = _quantize_rows_q4(bf16_bits_to_f32(L["up"][e]))
        rows[e, :, 2] = _quantize_rows_q4(np.ascontiguousarray(bf16_bits_to_f32(L["down"][e]).T))
    return {"rows": rows, "router": L["router"]}


def make_tokens(wl: Workload, n: int | None = None, seed_offset: int = 0) -> np.ndarray:
    """Decode-time hidden states x, float32 [n][H]."""
    n = wl.n_tokens if n is None else n
    rng = _rng(wl.token_seed + seed_offset, _STREAM_TOK)
    x = rng.standard_normal((n, wl.shape.hidden), dtype=np.float32)
    if wl.x_outlier_dims:
        x[:, x_outlier_dims(wl)] *= np.float32(wl.x_outlier_mult)
    return x


def make_routing_inputs(wl: Workload, n: int, seed_offset: int = 0):
    """Random routing for a decode call when no router is involved.

    expert_ids: int32 [n][top], distinct per token.
    gate_w:     float32 [n][top], positive, summing to one per token,
                sorted descending (the shape a softmax top-k router produces).
    """
    s = wl.shape
    rng = _rng(wl.token_seed + seed_offset, _STREAM_IDS)
    ids = np.stack([rng.choice(s.n_experts, size=s.top, replace=False) for _ in range(n)])
    rng2 = _rng(wl.token_seed + seed_offset, _STREAM_GW)
    g = rng2.dirichlet(np.ones(s.top), size=n)
    g = -np.sort(-g, axis=1)
    return ids.astype(np.int32), g.astype(np.float32)
