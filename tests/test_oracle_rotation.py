"""Pins for the block-128 randomized Hadamard rotation (closed forms, library routine)."""
import numpy as np
import scipy.linalg

from oracle.rotation import (SQRT128, rotate_rows, rotate_x_f64, rotate_x_f32_unscaled,
                             rotation_matrix, sign_vector, splitmix64_stream, sylvester_hadamard)


def test_sylvester_equals_scipy_and_recursion():
    h = sylvester_hadamard(128)
    assert np.array_equal(h, scipy.linalg.hadamard(128))
    h64 = sylvester_hadamard(64)
    assert np.array_equal(h, np.block([[h64, h64], [h64, -h64]]))
    assert np.array_equal(h @ h.T, 128 * np.eye(128))


def test_rotation_orthogonal_and_preserves_dot_products():
    sig = sign_vector(12345, 512)
    r = rotation_matrix(sig)
    assert np.abs(r.T @ r - np.eye(512)).max() < 1e-15
    rng = np.random.default_rng(0)
    g, x = rng.standard_normal(512), rng.standard_normal(512)
    rg = rotate_rows(g, sig).reshape(-1) / SQRT128
    rx = rotate_x_f64(x, sig).reshape(-1)
    assert abs(rg @ rx - g @ x) <= 1e-12 * np.abs(g).sum() * np.abs(x).max()
    # the fast form equals the dense matrix
    assert np.abs(r @ x - rx).max() < 1e-13


def test_signs_are_per_coordinate_and_balanced():
    sig = sign_vector(0x5EED, 4096)
    assert set(np.unique(sig).tolist()) == {-1.0, 1.0}
    assert abs(sig.mean()) < 0.06
    # blocks carry different sign patterns
    assert not np.array_equal(sig[:128], sig[128:256])


def test_splitmix64_reference_outputs():
    # first outputs of the SplitMix64 reference generator (Steele, Lea, Flood 2014)
    assert splitmix64_stream(0, 5) == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F,
                                       0xF88BB8A8724C81EC, 0x1B39896A51A8749B]
    assert splitmix64_stream(1234567, 3) == [0x599ED017FB08FC85, 0x2C73F08458540FA5,
                                             0x883EBCE5A3F27C77]


def test_f32_butterfly_exact_on_integers_and_close_otherwise():
    rng = np.random.default_rng(1)
    sig = sign_vector(99, 256)
    xi = rng.integers(-1000, 1000, 256).astype(np.float32)
    v = rotate_x_f32_unscaled(xi, sig)
    exact = (sylvester_hadamard(128) @ (xi.astype(np.float64) * sig).reshape(2, 128).T).T
    assert np.array_equal(v.astype(np.float64), exact)
    x = rng.standard_normal(256).astype(np.float32)
    v = rotate_x_f32_unscaled(x, sig).astype(np.float64)
    ref = rotate_rows(x.astype(np.float64), sig)
    assert np.abs(v - ref).max() < 1e-5 * np.abs(ref).max()
    assert rotate_x_f32_unscaled(x, sig).dtype == np.float32
