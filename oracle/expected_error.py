"""Ranking by expected squared output error, for budgets from 28.7% on.  (Oracle.)

What the pages fix ([zh §方法步骤详情] decode step (2)): from the 28.7% read
budget on, the reader reads the whole sketch (all 128 coordinates of every
block) and ranks the candidate channels with the help of the stored block
quantisation error rho_b by the expected squared output error that skipping
each of them would cause.  Below that budget the partial screen and the
output-unit score s_j = w_j ||d_j|| |phi(g_hat_j) v_hat_j| are used.

Reading of the open points (the library implements the same):
  * Sketch error model.  Per (row, block) the quantisation error of the
    normalised rotated row, e_b = r_b - alpha_b c_b, has mean square rho_b per
    coordinate (rho's definition, see the sketch module).  Taking its
    direction as uncorrelated with the rotated token block, the error of the
    full-sketch estimate g^T x - g_hat has variance
        var_g = sum_b rho_b ||x_b||^2
    because the block rotation is orthogonal, ||(R x)_b|| = ||x_b||.  The up
    rows' rho give var_v the same way.
  * Activation.  a_j = phi(g_j^T x)(v_j^T x) is estimated at (g_hat, v_hat)
    with independent errors of those variances, to first order (delta
    method): E[a] ~= p = phi(g_hat) v_hat and
        Var[a] ~= (phi'(g_hat) v_hat)^2 var_g + phi(g_hat)^2 var_v,
    with phi' the SiLU derivative sigma(z) (1 + z (1 - sigma(z))).
  * Error of skipping j.  Its output contribution w_j a_j d_j is left out:
    E||w_j a_j d_j||^2 = w_j^2 ||d_j||^2 (p_j^2 + Var[a_j]).  Candidates are
    ranked by the square root, in output units,
        e_j = w_j ||d_j|| sqrt(p_j^2 + Var[a_j]),
    top k by e_j, ties to the lower candidate index.  With var = 0 this is the
    low-budget score s_j.  The recovery of the skipped set is not credited
    in the ranking; a second reading would subtract what U b_j restores,
    w_j^2 (p_j^2 (||d_j||^2 - ||b_j||^2) + Var[a_j] ||d_j||^2).
  * The rest of the decode is unchanged: the exact part over the kept set
    and the recovery U sum_S w_j b_j p_j with p_j = phi(g_hat_j) v_hat_j.

Pins (tests/test_oracle_expected_error.py): phi' against a central
difference of SiLU; var_g against the empirical mean squared error of the
full-sketch estimate over many random tokens (a units or index mistake moves
it by a factor); Var[a] against Monte Carlo sampling of phi(g) v; e_j = s_j
when the variances are zero; the kept set with k = all reproduces the dense
MLP.
"""
import numpy as np


def silu_grad(z):
    """d/dz of z sigma(z): sigma(z) (1 + z (1 - sigma(z)))."""
    z = np.asarray(z, dtype=np.float64)
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def block_norms2(x, block=128):
    """||x_b||^2 per 128-block of the token (float64, summed in index order)."""
    xb = np.asarray(x, dtype=np.float32).astype(np.float64).reshape(-1, block)
    acc = np.zeros(xb.shape[0])
    for i in range(block):
        acc = acc + xb[:, i] * xb[:, i]
    return acc


def sketch_variance(rho, xb2):
    """var = sum_b rho[..., b] ||x_b||^2, summed in block order.

    rho: [..., nblk] (stored fp16 values as float64); xb2: [nblk]."""
    rho = np.asarray(rho, dtype=np.float64)
    acc = np.zeros(rho.shape[:-1])
    for b in range(rho.shape[-1]):
        acc = acc + rho[..., b] * xb2[b]
    return acc


def activation_variance(ghat, vhat, var_g, var_v):
    """First-order Var[phi(g) v] at (g_hat, v_hat) with independent errors."""
    ghat = np.asarray(ghat, dtype=np.float64)
    vhat = np.asarray(vhat, dtype=np.float64)
    s = 1.0 / (1.0 + np.exp(-ghat))
    phi = ghat * s
    dphi = silu_grad(ghat)
    return (dphi * vhat) ** 2 * var_g + phi ** 2 * var_v


def expected_error_score(ghat, vhat, var_g, var_v, w, dnorm):
    """e_j = w_j ||d_j|| sqrt(p_j^2 + Var[a_j]) with p_j = phi(g_hat) v_hat."""
    ghat = np.asarray(ghat, dtype=np.float64)
    p = ghat / (1.0 + np.exp(-ghat)) * np.asarray(vhat, dtype=np.float64)
    va = activation_variance(ghat, vhat, var_g, var_v)
    return np.asarray(w, dtype=np.float64) * np.asarray(dnorm, dtype=np.float64) * np.sqrt(p * p + va)
