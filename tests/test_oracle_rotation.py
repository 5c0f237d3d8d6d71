"""Pins for the block-128 randomized Hadamard rotation (closed forms, library routine)."""
import numpy as np
import scipy.linalg

from oracle.rotation import (SQRT128, rotate_rows, rotate_x_f64, rotation_matrix,
                             sign_vector, splitmix64_stream, sylvester_hadamard)


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


def test_one_hot_block_rotates_to_signed_constant():
    # R e_i = sigma_i h_i / sqrt(128): every coordinate of the block has
    # magnitude 1/sqrt(128), with the signs of column i of H_128 times sigma_i
    sig = sign_vector(99, 256)
    h = sylvester_hadamard(128)
    for i in (0, 1, 77, 128, 200, 255):
        x = np.zeros(256)
        x[i] = 1.0
        rx = rotate_x_f64(x, sig)
        b, c = divmod(i, 128)
        assert np.array_equal(np.abs(rx[b]), np.full(128, 1.0 / SQRT128))
        assert np.array_equal(np.sign(rx[b]), sig[i] * h[:, c])
        assert not rx[1 - b].any()
