"""Pins for the expected-error ranking of budgets from 28.7% on
([zh §方法步骤详情] decode step (2)): the whole sketch is read and candidates
are ranked with rho_b by the expected squared output error of skipping.

Each test names what it checks and which plausible mistake would fail it.
"""
import numpy as np
import pytest

from oracle import OracleReader, dense_moe, route, topk_desc
from oracle.dense import silu
from oracle.expected_error import (activation_variance, block_norms2, expected_error_score,
                                   sketch_variance, silu_grad)
from oracle.numerics import bf16_to_f64
from synth import f32_to_bf16_bits, make_layer, make_tokens, workload

TINY = workload("tiny")
S = TINY.shape


def test_silu_grad_matches_central_difference():
    # phi'(z) = sigma(z)(1 + z(1 - sigma(z))) against (phi(z+h) - phi(z-h)) / 2h:
    # a sign or a missing factor in the derivative fails
    z = np.linspace(-30.0, 30.0, 1201)
    h = 1e-5
    fd = (silu(z + h) - silu(z - h)) / (2 * h)
    assert np.max(np.abs(fd - silu_grad(z))) < 1e-8


def test_block_norms_are_sums_of_squares():
    x = np.arange(256, dtype=np.float32) / 16.0
    got = block_norms2(x)
    ref = [float(np.sum(x[:128].astype(np.float64) ** 2)), float(np.sum(x[128:].astype(np.float64) ** 2))]
    assert np.allclose(got, ref, rtol=1e-15)


@pytest.fixture(scope="module")
def skewed_layer():
    # weights whose second block is 5x larger (so its rho is ~25x larger) and
    # up rows 3x larger than gate rows: swapping blocks or halves moves the
    # predicted variance by a large factor
    rng = np.random.default_rng(11)
    E, I, H = 8, 64, 256
    def rows(scale):
        w = rng.normal(0.0, 0.02, size=(E, I, H)) * scale
        w[:, :, 128:] *= 5.0
        return f32_to_bf16_bits(w.astype(np.float32))
    gate, up = rows(1.0), rows(3.0)
    down = f32_to_bf16_bits(rng.normal(0.0, 0.02, size=(E, H, I)).astype(np.float32))
    o = OracleReader(H, E, I, E, gate, up, down, n_screen=128, rank=8)
    return o, gate, up


def test_sketch_variance_matches_empirical_sketch_error(skewed_layer):
    # var_g = sum_b rho_b ||x_b||^2 against the mean squared error of the
    # full-sketch estimate g_hat over many random tokens, with g^T x from the
    # native rows.  Tokens have block norms 5:1 so a block swap, the wrong half,
    # or a factor of 128 in rho's units all fail.
    o, gate, up = skewed_layer
    rng = np.random.default_rng(12)
    E, I, H = o.E, o.I, o.H
    ids = np.arange(E)
    n = 300
    err2 = np.zeros((2, E, I))
    pred = np.zeros((2, E, I))
    G, V = bf16_to_f64(gate), bf16_to_f64(up)
    for _ in range(n):
        x = rng.normal(size=H)
        x[:128] *= 5.0
        x = x.astype(np.float32)
        _, sel = o.select(x)
        gh, vh = o.screen(x, ids, sel)
        x64 = x.astype(np.float64)
        err2[0] += (G @ x64 - gh) ** 2
        err2[1] += (V @ x64 - vh) ** 2
        xb2 = block_norms2(x)
        pred[0] += sketch_variance(o.rho[:, :, 0, :].transpose(0, 2, 1), xb2)
        pred[1] += sketch_variance(o.rho[:, :, 1, :].transpose(0, 2, 1), xb2)
    for m in range(2):
        ratio = err2[m] / pred[m]
        assert abs(err2[m].sum() / pred[m].sum() - 1.0) < 0.03, m
        assert np.mean(np.abs(ratio - 1.0) < 0.3) > 0.95, m


def test_activation_variance_matches_monte_carlo():
    # first-order Var[phi(g) v] against sampling with small independent
    # errors: dropping v_hat from the phi' term or phi from the v term fails
    rng = np.random.default_rng(13)
    for gh, vh in [(0.7, -1.3), (-2.0, 0.4), (3.5, 2.0), (-0.2, 5.0)]:
        vg, vv = (0.02 * abs(gh) + 1e-3) ** 2, (0.02 * abs(vh) + 1e-3) ** 2
        g = gh + rng.normal(size=400_000) * np.sqrt(vg)
        v = vh + rng.normal(size=400_000) * np.sqrt(vv)
        emp = np.var(silu(g) * v)
        ref = activation_variance(gh, vh, vg, vv)
        assert abs(emp / ref - 1.0) < 0.03, (gh, vh, emp, ref)


def test_zero_variance_reduces_to_output_unit_score():
    rng = np.random.default_rng(14)
    gh, vh = rng.normal(size=50) * 3, rng.normal(size=50) * 3
    w, dn = rng.uniform(0.05, 1.0, 50), rng.uniform(0.1, 2.0, 50)
    e = expected_error_score(gh, vh, 0.0, 0.0, w, dn)
    s = w * dn * np.abs(silu(gh) * vh)
    assert np.allclose(e, s, rtol=1e-14, atol=0.0)


def test_variance_only_raises_the_score():
    rng = np.random.default_rng(15)
    gh, vh = rng.normal(size=200) * 2, rng.normal(size=200) * 2
    w, dn = rng.uniform(0.05, 1.0, 200), rng.uniform(0.1, 2.0, 200)
    s = expected_error_score(gh, vh, 0.0, 0.0, w, dn)
    e = expected_error_score(gh, vh, 0.01, 0.02, w, dn)
    assert np.all(e >= s)
    assert np.any(e > s)


@pytest.fixture(scope="module")
def tiny_full():
    layer = make_layer(TINY)
    o = OracleReader(S.hidden, S.n_experts, S.inter, S.top, layer["gate"], layer["up"],
                     layer["down"], layer["router"], n_screen=128)
    return layer, o


def test_expected_error_keep_all_equals_dense(tiny_full):
    layer, o = tiny_full
    for x in make_tokens(TINY, 3):
        ids, w, _ = route(layer["router"], x, S.top)
        w32 = w.astype(np.float32)
        out = o.decode(x, ids, w32, S.n_cand, ranking="expected_error")
        ref = dense_moe(layer["gate"], layer["up"], layer["down"], x, ids, w32)
        assert np.linalg.norm(out["y"] - ref) <= 1e-12 * np.linalg.norm(ref)


def test_expected_error_kept_set_is_the_stable_top_k_of_e(tiny_full):
    # the kept set is the k largest e_j, ties to the lower candidate index,
    # and e_j >= the output-unit score of the same candidate
    layer, o = tiny_full
    for x in make_tokens(TINY, 4):
        ids, w, _ = route(layer["router"], x, S.top)
        w32 = w.astype(np.float32)
        ee = o.decode(x, ids, w32, 23, ranking="expected_error")
        sc = o.decode(x, ids, w32, 23, ranking="score")
        order = sorted(range(S.n_cand), key=lambda c: (-ee["score"].reshape(-1)[c], c))
        assert sorted(order[:23]) == ee["kept"].tolist()
        assert np.all(ee["score"] >= sc["score"] * (1 - 1e-12))
        np.testing.assert_array_equal(topk_desc(ee["score"].reshape(-1), 23), ee["kept"])


def test_expected_error_needs_the_whole_sketch():
    layer = make_layer(TINY)
    o = OracleReader(S.hidden, S.n_experts, S.inter, S.top, layer["gate"], layer["up"],
                     layer["down"], n_screen=80)
    x = make_tokens(TINY, 1)[0]
    with pytest.raises(AssertionError):
        o.decode(x, np.arange(S.top), np.ones(S.top, np.float32), 10, ranking="expected_error")
