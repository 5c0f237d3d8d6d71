"""Layer-wide low-rank recovery basis.  (Oracle: test infrastructure.)

The pages stack the down-projection columns of every expert in a layer, take
the top-32 left singular vectors U, and store b_j = U^T d_j, so U b_j ~= d_j
stands in for the down column of a skipped channel
([zh §前置知识 / 低秩恢复]; [zh §方法步骤详情] load step (3); [ko §어떻게 쓰나]).

Reading: D_all = [D_0 | ... | D_{E-1}] (H x E*I, not centred).  U = the
eigenvectors of the float64 Gram D_all D_all^T (accumulated expert by expert
with BLAS dsyrk) for its ``rank`` largest eigenvalues (numpy.linalg.eigh),
which are the top left singular vectors;
b = U^T D_all in float64.  Storage rounding (fp16) is applied by the caller.
U is unique only up to a rotation inside eigenvalue clusters and column
signs; every use of it goes through U b, which is invariant.

Pins (tests/test_oracle_reader.py): U from eigh spans the same space as the
left singular vectors from numpy.linalg.svd; with rank = H the recovery term
equals the exact skipped contribution.
"""
import numpy as np
from scipy.linalg.blas import dsyrk

from .numerics import weights_f64


def recovery_basis(down_bits: np.ndarray, rank: int):
    """down_bits: bf16 [E][H][I].  Returns (U [H][rank], b [E][I][rank]) float64."""
    e, h, i = down_bits.shape
    # the Gram matrix sum_e D_e D_e^T, upper triangle (BLAS dsyrk: the same
    # products as D_e @ D_e.T, half of them)
    gram = np.zeros((h, h), order="F")
    for ex in range(e):
        d = weights_f64(down_bits[ex])  # [H][I]
        gram = dsyrk(1.0, d, beta=1.0, c=gram, overwrite_c=True)
    vals, vecs = np.linalg.eigh(gram, UPLO="U")
    order = np.argsort(-vals, kind="stable")[:rank]
    u = vecs[:, order]
    b = np.empty((e, i, rank))
    for ex in range(e):
        b[ex] = (u.T @ weights_f64(down_bits[ex])).T
    return u, b
