"""Block-128 randomized Hadamard rotation.  (Oracle: test infrastructure.)

The reader rotates every gate/up row and the token x with a random Hadamard
matrix R applied per 128-coordinate block; R is orthogonal, so
g^T x = (R g)^T (R x) ([zh §前置知识 / Hadamard旋转与三元Sketch];
[zh §方法步骤详情] load step (1) and decode step (1); [ko §어떻게 쓰나]).

Reading of what the pages leave open (the library implements the same):
  * H_128 is the Sylvester Hadamard matrix in natural order:
    H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]].
  * R = blockdiag(H_128, ..., H_128) . diag(sigma) / sqrt(128), one sign per
    hidden coordinate, one R per layer shared by every expert (x is rotated
    once per token and layer).
  * sigma_i = -1 if the top bit of output i (i = 0, 1, ...) of the SplitMix64
    generator seeded with ``rot_seed`` is set, else +1.  SplitMix64 is the
    published generator of Steele, Lea and Flood (OOPSLA 2014): the state
    advances by 0x9E3779B97F4A7C15 and each output is the state passed
    through the finalizer  z ^= z>>30; z *= 0xBF58476D1CE4E5B9;
    z ^= z>>27; z *= 0x94D049BB133111EB; z ^= z>>31  (all mod 2^64).
  * The partial screen ranks coordinates by |(R x)_i|, evaluated here in
    float64 (the module reader takes the ranking on these values; ties go to
    the lower index).

Pins (tests/test_oracle_rotation.py): H_128 equals scipy.linalg.hadamard(128)
and the explicit recursion; R^T R = I; g^T x = (Rg)^T (Rx); R x of a one-hot
block is +-1/sqrt(128) everywhere; SplitMix64's first outputs for seed 0 equal
the generator's published reference values.
"""
import numpy as np

SQRT128 = 11.313708498984761  # sqrt(128) rounded to the nearest float64
_M64 = (1 << 64) - 1


def splitmix64_stream(seed: int, n: int) -> list:
    """First n outputs of SplitMix64 seeded with ``seed`` (Python ints)."""
    state = seed & _M64
    out = []
    for _ in range(n):
        state = (state + 0x9E3779B97F4A7C15) & _M64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
        z = z ^ (z >> 31)
        out.append(z)
    return out


def sign_vector(seed: int, hidden: int) -> np.ndarray:
    """sigma in {+1, -1}^hidden as float64."""
    return np.array([-1.0 if (z >> 63) else 1.0 for z in splitmix64_stream(seed, hidden)])


def sylvester_hadamard(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order n (a power of two), natural order."""
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    assert h.shape[0] == n
    return h


def rotation_matrix(sigma: np.ndarray, block: int = 128) -> np.ndarray:
    """Dense R = blockdiag(H_block) diag(sigma) / sqrt(block) (for small checks)."""
    hid = sigma.shape[0]
    hb = sylvester_hadamard(block)
    r = np.zeros((hid, hid))
    for b in range(hid // block):
        sl = slice(b * block, (b + 1) * block)
        r[sl, sl] = hb * sigma[None, sl]
    return r / np.sqrt(float(block))


def rotate_rows(w: np.ndarray, sigma: np.ndarray, block: int = 128) -> np.ndarray:
    """Un-normalised rotated rows u = H_128 (sigma * w) per block, float64.

    ``w`` has shape [..., H]; the result has shape [..., H/128, 128].
    (R w) = u / sqrt(128).
    """
    hid = w.shape[-1]
    nb = hid // block
    ws = (np.asarray(w, dtype=np.float64) * sigma).reshape(w.shape[:-1] + (nb, block))
    hb = sylvester_hadamard(block)  # symmetric
    return ws @ hb


def rotate_x_f64(x: np.ndarray, sigma: np.ndarray, block: int = 128) -> np.ndarray:
    """R x in float64, shape [..., H/128, 128]."""
    return rotate_rows(x, sigma, block) / SQRT128
