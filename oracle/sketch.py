"""Ternary sketch of the rotated gate/up rows and its byte layout.  (Oracle.)

What the pages fix ([zh §前置知识 / Hadamard旋转与三元Sketch]; [zh §方法步骤详情]
load step (1); [zh §技术新颖性]; [ko §어떻게 쓰나]): after rotation, every
(row, 128-block) is stored as codes in {-1, 0, 1}, one FP16 scale and the
block's mean squared quantisation error rho_b; the codes follow Ternary Weight
Networks; a 256-byte BF16 block shrinks to about 30 bytes; the whole sketch is
about 7% of the BF16 checkpoint.

Reading of the open points (the library implements the same):
  * Ternary Weight Networks rule on the un-normalised rotated block u (128
    values): S = sum_i |u_i| summed in index order in float64; code
    c_i = sign(u_i) if 1280 * |u_i| > 7 * S, else 0 (the threshold
    0.7 * mean|u| written with multiplications only, so both sides round
    identically).
  * Scale alpha = fp16( A / (n * sqrt(128)) ) with A = sum of |u_i| over the
    nonzero codes (index order), n = their count; alpha = 0 when n = 0.  The
    division by sqrt(128) puts alpha in the units of the normalised rotated
    row R g, so  (R g)_i ~= alpha * c_i.
  * rho = fp16( sum_i (r_i - alpha * c_i)^2 / 128 ) with r_i = u_i / sqrt(128),
    summed in index order: the block's mean squared quantisation error in the
    same units.  (Stored; the low-budget decode path does not read it.)
  * Byte layout, coordinate-major so that a partial screen can read one
    coordinate's codes for every channel of an expert at once: one unit per
    (expert, block, coordinate).  Inside a unit, the gate codes of channels
    0..I-1 come first, five per byte, byte q = sum_{t<5} (c_{5q+t} + 1) 3^t
    (channels >= I count as code 0); the gate half is zero-padded to
    Lp = roundup(ceil(I/5), 16) bytes; the up half follows at byte Lp in the
    same form; the unit is zero-padded to roundup(2 Lp, 32) bytes, a whole
    number of 32-byte sectors.  Units are ordered [expert][block][coordinate].
    Unit sizes: 32 B (I = 64), 320 B (I = 768), 640 B (I = 1536).

Pins (tests/test_oracle_sketch.py): worked special cases derived from the
definition (one-hot block, Hadamard-row block, zero block), the threshold
invariant on random blocks, hand-worked bytes (tests/golden/pack_bytes.json),
pack/unpack round trip, bytes per block vs the pages' ~30 B.
"""
import numpy as np

from .numerics import f64_to_f16_bits, f16_bits_to_f64
from .rotation import SQRT128


def ternarize_blocks(u: np.ndarray):
    """TWN codes, scale and rho for blocks u[..., 128] (float64, un-normalised).

    Returns (codes int8 [..., 128], alpha fp16 bits [...], rho fp16 bits [...]).
    """
    u = np.asarray(u, dtype=np.float64)
    nblk = u.shape[-1]
    # coordinate-major copies, so that each index-ordered sum below walks
    # contiguous slices (the same additions in the same order)
    uT = np.ascontiguousarray(np.moveaxis(u, -1, 0))
    auT = np.abs(uT)
    s = np.zeros(u.shape[:-1])
    for i in range(nblk):
        s = s + auT[i]
    keepT = 1280.0 * auT > 7.0 * s
    codesT = (np.sign(uT) * keepT).astype(np.int8)
    n = keepT.sum(axis=0)
    a = np.zeros(u.shape[:-1])
    for i in range(nblk):
        a = a + np.where(keepT[i], auT[i], 0.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        alpha64 = np.where(n > 0, a / (n * SQRT128), 0.0)
    alpha_bits = f64_to_f16_bits(alpha64)
    alpha = f16_bits_to_f64(alpha_bits)
    rT = uT / SQRT128
    acc = np.zeros(u.shape[:-1])
    for i in range(nblk):
        d = rT[i] - alpha * codesT[i]
        acc = acc + d * d
    rho_bits = f64_to_f16_bits(acc / 128.0)
    codes = np.ascontiguousarray(np.moveaxis(codesT, 0, -1))
    return codes, alpha_bits, rho_bits


def unit_geometry(inter: int):
    """(half_bytes Lp, unit_bytes) of one coordinate unit for I channels."""
    lp = -(-inter // 5)
    lp = -(-lp // 16) * 16
    unit = -(-(2 * lp) // 32) * 32
    return lp, unit


def _pack_half(codes_ci: np.ndarray, lp: int) -> np.ndarray:
    """codes [..., I] in {-1,0,1} -> bytes [..., lp] (base 3, five codes per byte)."""
    inter = codes_ci.shape[-1]
    nbytes = -(-inter // 5)
    # digits fit in uint8 and so does every byte (at most 2 * 121 = 242)
    t = np.empty(codes_ci.shape[:-1] + (nbytes * 5,), dtype=np.uint8)
    t[..., inter:] = 1  # code 0 -> digit 1
    t[..., :inter] = (codes_ci + 1).astype(np.uint8)
    t = t.reshape(codes_ci.shape[:-1] + (nbytes, 5))
    q = t[..., 0] + np.uint8(3) * t[..., 1] + np.uint8(9) * t[..., 2] + \
        np.uint8(27) * t[..., 3] + np.uint8(81) * t[..., 4]
    out = np.zeros(codes_ci.shape[:-1] + (lp,), dtype=np.uint8)
    out[..., :nbytes] = q
    return out


def pack_units(codes_gate: np.ndarray, codes_up: np.ndarray) -> np.ndarray:
    """Coordinate-major codes [..., I] (gate and up) -> units [..., unit_bytes] uint8."""
    inter = codes_gate.shape[-1]
    lp, unit = unit_geometry(inter)
    out = np.zeros(codes_gate.shape[:-1] + (unit,), dtype=np.uint8)
    out[..., :lp] = _pack_half(codes_gate, lp)
    out[..., lp:2 * lp] = _pack_half(codes_up, lp)
    return out


def unpack_units(units: np.ndarray, inter: int):
    """Inverse of pack_units: units [..., unit_bytes] -> (gate, up) codes [..., I] int8."""
    lp, unit = unit_geometry(inter)
    assert units.shape[-1] == unit
    nbytes = -(-inter // 5)
    res = []
    for h in range(2):
        q = units[..., h * lp:h * lp + nbytes].astype(np.int64)
        digits = []
        for _ in range(5):
            digits.append(q % 3)
            q = q // 3
        t = np.stack(digits, axis=-1).reshape(units.shape[:-1] + (nbytes * 5,))
        res.append((t[..., :inter] - 1).astype(np.int8))
    return res[0], res[1]
