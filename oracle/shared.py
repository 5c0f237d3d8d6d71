"""Batch-shared channel selection.  (Oracle: test infrastructure.)

The pages name selecting channels jointly for the whole batch as the way to
keep the reader's gain at larger batches, and leave it as future work
([zh §未来方向] direction (1); [ko §전제와 한계], last paragraph).  They give
no formula; this module fixes the plainest reading that the per-token method
supports and the library implements the same:

  * candidates: the channels of the batch's distinct routed experts, union
    candidate u * I + j for the u-th distinct expert in ascending id order;
  * batch score of a candidate: the sum, over the (token, slot) pairs routed
    to its expert (token-major, slot order), of the per-token output-unit
    score w ||d_j|| |phi(g_hat_j) v_hat_j| -- the total magnitude of the
    channel's contributions to the batch's outputs;
  * keep exactly the k highest batch scores (ties to the lower union
    candidate), so each kept channel's native rows are read once for the
    batch and give the exact a_j of every token routed to its expert;
  * every token recovers its own skipped channels with its own p_j:
    z_t = sum over its routed (slot, j) not kept of w p_j b_j, y_t = exact
    part + U z_t.

With one token the union is its routed experts in ascending id order instead
of slot order, the batch scores are the token's scores, and the kept set,
hence y, is the per-token decode's.

Pins (tests/test_oracle_shared.py): a batch of one keeps the per-token set
and gives its y (within float64 rounding: the sums run slot by slot); two
copies of a token with the same routing keep the per-token set and give its
y; k = every union candidate gives each token's dense gated MLP; k = 0 gives
each token its recovery alone; a kept channel of an expert two tokens share
is exact for both and its batch score is the sum of theirs; brute force over
all k-subsets on a tiny batch maximises the summed batch score.
"""
import numpy as np

from .dense import silu
from .numerics import weights_f64
from .topk import topk_desc


def decode_shared(oracle, X, IDS, W, k, kept=None):
    """Batch-shared decode with an OracleReader.  X [B][H], IDS [B][top],
    W [B][top], k kept union candidates.  Returns a dict: "experts" (the
    union, ascending), "bscore" [u][I], "kept" (union candidates, ascending),
    and per token "y", "y_exact", "y_rec", "p".  kept, when given, replaces
    the top-k (for comparisons where neighbouring batch scores tie within
    rounding)."""
    X = np.asarray(X, dtype=np.float32)
    IDS = np.asarray(IDS, dtype=np.int64)
    W = np.asarray(W, dtype=np.float32).astype(np.float64)
    B, top = IDS.shape
    I, H = oracle.I, oracle.H
    experts = np.unique(IDS)
    uix = {int(e): u for u, e in enumerate(experts.tolist())}
    # decode steps (1)-(2) per token: screen estimates and p = phi(g_hat) v_hat
    P = []
    for t in range(B):
        _, sel = oracle.select(X[t])
        ghat, vhat = oracle.screen(X[t], IDS[t], sel)
        P.append(silu(ghat) * vhat)
    # batch scores, token-major then slot order
    bscore = np.zeros((experts.size, I))
    for t in range(B):
        for s in range(top):
            e = int(IDS[t, s])
            dn = oracle.norms[oracle.ix([e])[0]].astype(np.float64)
            bscore[uix[e]] = bscore[uix[e]] + W[t, s] * dn * np.abs(P[t][s])
    if kept is None:
        kept = topk_desc(bscore.reshape(-1), min(int(k), bscore.size))
    else:
        kept = np.sort(np.asarray(kept, dtype=np.int64))
    kmask = np.zeros(bscore.size, dtype=bool)
    kmask[kept] = True
    kmask = kmask.reshape(experts.size, I)
    ys, yex, yrec = [], [], []
    for t in range(B):
        x64 = X[t].astype(np.float64)
        y_exact = np.zeros(H)
        z = np.zeros(oracle.rank)
        for s in range(top):
            e = int(IDS[t, s])
            km = kmask[uix[e]]
            j = np.nonzero(km)[0]
            if j.size:
                a = silu(weights_f64(oracle.gate[e, j]) @ x64) * (weights_f64(oracle.up[e, j]) @ x64)
                y_exact = y_exact + (W[t, s] * a) @ weights_f64(oracle.down[e][:, j]).T
            sk = np.nonzero(~km)[0]
            if sk.size:
                z = z + (W[t, s] * P[t][s][sk]) @ oracle.b[e, sk]
        y_rec = oracle.U @ z
        ys.append(y_exact + y_rec)
        yex.append(y_exact)
        yrec.append(y_rec)
    return {"experts": experts, "bscore": bscore, "kept": kept, "y": np.stack(ys),
            "y_exact": np.stack(yex), "y_rec": np.stack(yrec), "p": P}
