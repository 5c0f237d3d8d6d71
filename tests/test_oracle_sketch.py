"""Pins for the ternary sketch: worked special cases, invariants, hand-worked bytes."""
import json
import os

import numpy as np
import pytest

from oracle.numerics import f16_bits_to_f64, f64_to_f16_bits
from oracle.rotation import SQRT128, rotate_rows, sign_vector, sylvester_hadamard
from oracle.sketch import pack_units, ternarize_blocks, unit_geometry, unpack_units


def _f16(v):
    return float(f16_bits_to_f64(f64_to_f16_bits(v)))


@pytest.mark.parametrize("c,i", [(0.03125, 5), (-0.4375, 127), (0.0234375, 0)])
def test_one_hot_block(c, i):
    # w = c e_i: sigma only flips signs, so |u| = |c| at all 128 coordinates
    sig = sign_vector(3, 128)
    w = np.zeros(128)
    w[i] = c
    u = rotate_rows(w, sig)[0]
    assert np.array_equal(np.abs(u), np.full(128, abs(c)))
    codes, a_bits, r_bits = ternarize_blocks(u[None])
    assert np.array_equal(codes[0], np.sign(c * sig[i] * sylvester_hadamard(128)[:, i]))
    alpha = _f16(abs(c) / SQRT128)
    assert float(f16_bits_to_f64(a_bits[0])) == alpha
    assert float(f16_bits_to_f64(r_bits[0])) == _f16((abs(c) / SQRT128 - alpha) ** 2)


@pytest.mark.parametrize("c,k", [(0.0625, 3), (-0.01171875, 100)])
def test_hadamard_row_block(c, k):
    # w = c (sigma * row k of H_128): u = 128 c e_k, exactly one nonzero code
    sig = sign_vector(4, 128)
    w = c * sig * sylvester_hadamard(128)[k]
    u = rotate_rows(w, sig)[0]
    exp_u = np.zeros(128)
    exp_u[k] = 128 * c
    assert np.array_equal(u, exp_u)
    codes, a_bits, r_bits = ternarize_blocks(u[None])
    exp_c = np.zeros(128, dtype=np.int8)
    exp_c[k] = np.sign(c)
    assert np.array_equal(codes[0], exp_c)
    alpha = _f16(abs(c) * 128 / SQRT128)
    assert float(f16_bits_to_f64(a_bits[0])) == alpha
    assert float(f16_bits_to_f64(r_bits[0])) == _f16((abs(c) * 128 / SQRT128 - alpha) ** 2 / 128)


def test_zero_block():
    codes, a_bits, r_bits = ternarize_blocks(np.zeros((3, 128)))
    assert not codes.any() and not a_bits.any() and not r_bits.any()


def test_threshold_invariant_and_scale_bounds():
    rng = np.random.default_rng(5)
    u = rng.standard_normal((500, 128)) * rng.uniform(0.01, 3, (500, 1))
    u[:50, :3] *= 40  # outlier coordinates
    codes, a_bits, r_bits = ternarize_blocks(u)
    mean_abs = np.abs(u).mean(axis=1, keepdims=True)
    keep = codes != 0
    # 0.7 * mean|u| threshold (Ternary Weight Networks), sign preserved
    assert np.all(np.abs(u)[keep] > (0.7 * mean_abs * np.ones_like(u))[keep] * (1 - 1e-12))
    assert np.all(np.abs(u)[~keep] <= (0.7 * mean_abs * np.ones_like(u))[~keep] * (1 + 1e-12))
    assert np.all(np.sign(u)[keep] == codes[keep])
    # alpha is the mean kept magnitude in normalised units
    alpha = f16_bits_to_f64(a_bits)
    ref = np.array([np.abs(u[r])[keep[r]].mean() / SQRT128 for r in range(500)])
    assert np.allclose(alpha, ref, rtol=1e-3)
    # rho is the mean squared error of the normalised block
    rho = f16_bits_to_f64(r_bits)
    err = ((u / SQRT128 - alpha[:, None] * codes) ** 2).mean(axis=1)
    assert np.allclose(rho, err, rtol=2e-3, atol=2.0 ** -24)


def test_hand_worked_bytes(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "pack_bytes.json")))
    for case in g["cases"]:
        inter = case["inter"]
        lp, unit = unit_geometry(inter)
        assert (lp, unit) == (case["half_bytes"], case["unit_bytes"])
        gc = np.zeros(inter, np.int8) if case["gate"] == "zeros" else np.array(case["gate"], np.int8)
        uc = np.zeros(inter, np.int8) if case["up"] == "zeros" else np.array(case["up"], np.int8)
        b = pack_units(gc[None], uc[None])[0]
        exp = np.zeros(unit, np.uint8)
        for k, v in case.get("nonzero", {}).items():
            exp[int(k)] = v
        for lo, hi, v in case.get("nonzero_range", []):
            exp[lo:hi] = v
        assert np.array_equal(b, exp), (b, exp)


@pytest.mark.parametrize("inter", [1, 4, 5, 6, 64, 768, 1536])
def test_pack_roundtrip(inter):
    rng = np.random.default_rng(inter)
    g = rng.integers(-1, 2, (3, 4, inter)).astype(np.int8)
    u = rng.integers(-1, 2, (3, 4, inter)).astype(np.int8)
    units = pack_units(g, u)
    assert units.shape[-1] % 32 == 0
    g2, u2 = unpack_units(units, inter)
    assert np.array_equal(g, g2) and np.array_equal(u, u2)


def test_unit_sizes_of_the_evaluated_shapes():
    assert unit_geometry(64) == (16, 32)
    assert unit_geometry(768) == (160, 320)
    assert unit_geometry(1536) == (320, 640)
