"""Pins of the 4-bit record format (oracle/int4.py)."""
import numpy as np

from oracle.int4 import dequant_layer, dequant_record, record_bytes
from synth import LayerShape, make_layer, make_layer_q4, q4_row_bytes, workload, bf16_bits_to_f32


def test_record_size_matches_the_generator():
    for H in (128, 256, 2048, 4096):
        assert record_bytes(H) == q4_row_bytes(H)
    # 2048 weights: 1024 code bytes + 16 scales (32 B) + 16 zero points
    assert record_bytes(2048) == 1072


def test_hand_worked_record():
    # H = 128: one group.  Codes: weight 0 -> 3, weight 1 -> 12, weight 2 -> 0,
    # weight 3 -> 15, the rest 7.  Scale 0.5 (fp16 0x3800), zero point 7:
    # weights (3-7)*0.5 = -2, (12-7)*0.5 = 2.5, -3.5, 4, then 0.
    H = 128
    rec = np.zeros(record_bytes(H), dtype=np.uint8)
    rec[:64] = 7 | (7 << 4)
    rec[0] = 3 | (12 << 4)
    rec[1] = 0 | (15 << 4)
    rec[64:66] = [0x00, 0x38]  # fp16 0.5, little endian
    rec[66] = 7
    w = dequant_record(rec, H)
    assert w[:4].tolist() == [-2.0, 2.5, -3.5, 4.0]
    assert np.all(w[4:] == 0.0)


def test_generator_error_is_at_most_half_a_step():
    # the generator's records decode to the layer's weights within half a
    # quantisation step
    shape = LayerShape(hidden=256, n_experts=2, inter=3, top=1)
    wl = workload("tiny", shape=shape)
    L = make_layer_q4(wl)
    gate, up, down = dequant_layer(L["rows"], 256)
    assert gate.shape == (2, 3, 256) and up.shape == (2, 3, 256) and down.shape == (2, 256, 3)
    # quantisation error of round to nearest: at most half a step per weight
    src = make_layer(wl)
    g32 = bf16_bits_to_f32(src["gate"]).astype(np.float64)
    rec = L["rows"][:, :, 0]
    scale = np.ascontiguousarray(rec[..., 128:132]).view(np.float16).astype(np.float64)
    step = np.repeat(scale, 128, axis=-1)
    assert np.all(np.abs(gate - g32) <= 0.5 * step + 1e-12)
    d32 = bf16_bits_to_f32(src["down"]).astype(np.float64)
    assert np.abs(down - d32).max() <= 0.5 * np.repeat(
        np.ascontiguousarray(L["rows"][:, :, 2, 128:132]).view(np.float16).astype(np.float64), 128, -1).max()
