"""Comparison rules between the HIP reader and the oracle (shared by GPU tests).

Bars (the method's stated acceptance):
  * the rotated token before scaling and the screened coordinates: bit-exact
    (both sides take the ranking on the same float32 butterfly values);
  * g_hat, v_hat, scores: within 1e-5 relative to the vector's largest
    magnitude (float32 accumulation over at most 80*nblk terms vs float64);
  * kept sets: equal outside a relative band of 1e-4 around the oracle's k-th
    score (neighbouring scores closer than that may swap), size exactly k;
  * y: within 2e-3 relative L2 of the oracle's y recomputed on the library's
    kept set (float32 accumulation over BF16 weights vs float64).
"""
import numpy as np

EST_RTOL = 1e-5
KEPT_BAND = 1e-4
Y_RTOL = 2e-3


def rel_max_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.abs(ref).max()
    return float(np.abs(got - ref).max() / scale) if scale > 0 else float(np.abs(got).max())


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / n) if n > 0 else float(np.linalg.norm(got))


def check_kept(lib_kept, ref, k, band=KEPT_BAND):
    """lib_kept: library's kept candidates; ref: oracle decode dict."""
    lib = np.asarray(lib_kept, dtype=np.int64)
    assert lib.shape == (k,), (lib.shape, k)
    assert len(set(lib.tolist())) == k, "duplicate kept candidates"
    assert np.all(np.diff(lib) > 0), "kept list not ascending"
    if k == 0:
        return 0
    s = ref["score"].reshape(-1)
    sk = np.sort(s)[::-1][k - 1]
    diff = set(lib.tolist()) ^ set(ref["kept"].tolist())
    for c in diff:
        assert abs(s[c] - sk) <= band * max(sk, 1e-30), (
            f"candidate {c} differs outside the tie band: score {s[c]} vs k-th {sk}")
    return len(diff)


def check_token(lib, ref, oracle, x, ids, w, k, t=0):
    """Compare one token of a decode_debug result dict (numpy) with the oracle."""
    assert np.array_equal(lib["xrot"][t].reshape(ref["v32"].shape), ref["v32"]), "rotation differs"
    assert np.array_equal(lib["sel"][t].astype(np.int64), ref["sel"]), "screened coordinates differ"
    assert rel_max_err(lib["ghat"][t], ref["ghat"].reshape(-1)) <= EST_RTOL
    assert rel_max_err(lib["vhat"][t], ref["vhat"].reshape(-1)) <= EST_RTOL
    assert rel_max_err(lib["score"][t], ref["score"].reshape(-1)) <= 2 * EST_RTOL
    ndiff = check_kept(lib["kept"][t], ref, k)
    yref = ref["y"] if ndiff == 0 else oracle.decode(x, ids, w, k, kept=lib["kept"][t])["y"]
    err = rel_l2(lib["y"][t], yref)
    assert err <= Y_RTOL, f"y rel L2 {err}"
    return err, ndiff
