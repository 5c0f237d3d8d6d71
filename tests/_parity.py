"""Comparison rules between the HIP reader and the oracle (shared by GPU tests).

Bars (the method's stated acceptance):
  * the rotated token: the library's float32 butterfly values H_128 (sigma x)
    within the butterfly's rounding bound of the oracle's float64 R x times
    sqrt(128): seven roundings of partial sums of at most sum |x_b| each;
  * the screened coordinates: equal to the oracle's (the n_screen largest
    float64 |R x| per block, ties to the lower index) outside a tie band of
    twice that bound around the block's n_screen-th magnitude, exactly
    n_screen distinct ascending coordinates per block; when a band swap
    occurs, the oracle's later steps are recomputed on the library's
    coordinates before the next comparisons;
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
SQRT128 = 11.313708498984761
# relative rounding bound of the seven-stage float32 butterfly, per unit of
# sum |x_b| (7 roundings, unit roundoff 2^-24, with one spare)
XROT_BOUND = 8 * 2.0 ** -24


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


def xrot_tolerance(x, nblk):
    """Per-block absolute bound on |H_128 (sigma x)| evaluated in float32."""
    return XROT_BOUND * np.abs(np.asarray(x, dtype=np.float32).astype(np.float64)).reshape(nblk, 128).sum(1)


def check_xrot(lib_xrot, ref, x):
    """lib_xrot: the library's un-normalised rotation [H]; ref: oracle decode dict."""
    nblk = ref["xr"].shape[0]
    got = np.asarray(lib_xrot, dtype=np.float64).reshape(nblk, 128)
    tol = xrot_tolerance(x, nblk)
    err = np.abs(got - SQRT128 * ref["xr"]).max(axis=1)
    assert np.all(err <= tol), f"rotation outside the float32 bound: {err} > {tol}"


def check_sel(lib_sel, ref, x):
    """Screened coordinates: the library's vs the oracle's, outside the tie band.
    Returns the number of coordinates that differ (all inside the band)."""
    nblk, ns = ref["sel"].shape
    lib = np.asarray(lib_sel, dtype=np.int64).reshape(nblk, ns)
    band = 2.0 * xrot_tolerance(x, nblk) / SQRT128
    ndiff = 0
    for b in range(nblk):
        row = lib[b]
        assert np.all((row >= 0) & (row < 128)), "screened coordinate out of range"
        assert np.all(np.diff(row) > 0), "screened coordinates not ascending and distinct"
        mag = np.abs(ref["xr"][b])
        t = np.sort(mag)[::-1][ns - 1]
        diff = set(row.tolist()) ^ set(ref["sel"][b].tolist())
        for c in diff:
            assert abs(mag[c] - t) <= band[b], (
                f"block {b}: coordinate {c} differs outside the tie band: |Rx| {mag[c]} vs "
                f"{ns}-th {t} (band {band[b]})")
        ndiff += len(diff)
    return ndiff


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
    """Compare one token of a decode_debug result dict (numpy) with the oracle.
    Returns (y relative L2 error, kept-set differences)."""
    ranking = ref.get("ranking", "score")
    check_xrot(lib["xrot"][t], ref, x)
    lib_sel = lib["sel"][t].astype(np.int64)
    if check_sel(lib_sel, ref, x):
        ref = oracle.decode(x, ids, w, k, ranking=ranking, sel=lib_sel)
    assert rel_max_err(lib["ghat"][t], ref["ghat"].reshape(-1)) <= EST_RTOL
    assert rel_max_err(lib["vhat"][t], ref["vhat"].reshape(-1)) <= EST_RTOL
    assert rel_max_err(lib["score"][t], ref["score"].reshape(-1)) <= 2 * EST_RTOL
    ndiff = check_kept(lib["kept"][t], ref, k)
    yref = ref["y"] if ndiff == 0 else oracle.decode(x, ids, w, k, kept=lib["kept"][t], ranking=ranking,
                                                     sel=lib_sel)["y"]
    err = rel_l2(lib["y"][t], yref)
    assert err <= Y_RTOL, f"y rel L2 {err}"
    return err, ndiff
