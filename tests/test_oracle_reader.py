"""Pins for the oracle reader: identities the method must reduce to.

Each test names the special case and why a plausible mistake would fail it.
"""
import numpy as np
import pytest

from oracle import OracleReader, dense_moe, route
from oracle.dense import silu
from oracle.numerics import bf16_to_f64, f16_bits_to_f64
from oracle.rotation import SQRT128, rotation_matrix, sign_vector, sylvester_hadamard
from oracle.sketch import unpack_units
from synth import f32_to_bf16_bits, make_layer, make_tokens, workload

TINY = workload("tiny")
S = TINY.shape


@pytest.fixture(scope="module")
def tiny_layer():
    return make_layer(TINY)


def _reader(layer, **kw):
    return OracleReader(S.hidden, S.n_experts, S.inter, S.top, layer["gate"], layer["up"],
                        layer["down"], layer["router"], **kw)


@pytest.fixture(scope="module")
def tiny_reader(tiny_layer):
    return _reader(tiny_layer)


def _tokens(n=6):
    return make_tokens(TINY, n)


def test_keep_all_equals_dense_gated_mlp(tiny_layer, tiny_reader):
    # k = all candidates: no recovery, y is the textbook gated MLP
    for x in _tokens():
        ids, w, _ = route(tiny_layer["router"], x, S.top)
        w32 = w.astype(np.float32)
        out = tiny_reader.decode(x, ids, w32, S.n_cand)
        ref = dense_moe(tiny_layer["gate"], tiny_layer["up"], tiny_layer["down"], x, ids, w32)
        assert np.linalg.norm(out["y"] - ref) <= 1e-12 * np.linalg.norm(ref)
        assert not out["z"].any()


def test_full_rank_recovery_equals_skipped_contribution(tiny_layer):
    # rank = H and unrounded storage: U b_j = d_j, so recovery is exact
    r = _reader(tiny_layer, rank=S.hidden, storage="fp64")
    for x in _tokens(3):
        ids, w, _ = route(tiny_layer["router"], x, S.top)
        out = r.decode(x, ids, w, 23)
        kept = set(out["kept"].tolist())
        ref = np.zeros(S.hidden)
        for c in range(S.n_cand):
            if c in kept:
                continue
            s, j = divmod(c, S.inter)
            e = ids[s]
            ref += np.float64(np.float32(w[s])) * out["p"][s, j] * bf16_to_f64(tiny_layer["down"][e][:, j])
        assert np.linalg.norm(out["y_rec"] - ref) <= 1e-10 * np.linalg.norm(ref)


def test_rank32_basis_spans_top_left_singular_vectors(tiny_reader, tiny_layer):
    d_all = np.concatenate([bf16_to_f64(tiny_layer["down"][e]) for e in range(S.n_experts)], axis=1)
    u_svd = np.linalg.svd(d_all, full_matrices=False)[0][:, :32]
    p1 = tiny_reader.U64 @ tiny_reader.U64.T
    p2 = u_svd @ u_svd.T
    assert np.abs(p1 - p2).max() < 1e-8
    # b = U^T d in float64 before rounding
    assert np.allclose(tiny_reader.b64[3, 5], tiny_reader.U64.T @ d_all[:, 3 * S.inter + 5])


def test_keep_none_is_pure_recovery(tiny_layer, tiny_reader):
    x = _tokens(1)[0]
    ids, w, _ = route(tiny_layer["router"], x, S.top)
    out = tiny_reader.decode(x, ids, w, 0)
    assert not out["y_exact"].any()
    z = sum(np.float64(np.float32(w[s])) * out["p"][s, j] * tiny_reader.b[ids[s], j]
            for s in range(S.top) for j in range(S.inter))
    assert np.allclose(out["z"], z, rtol=1e-12, atol=1e-15)
    assert np.allclose(out["y"], tiny_reader.U @ z, rtol=1e-12, atol=1e-15)


def test_partial_screen_is_exact_when_rx_lives_on_the_screened_coordinates(tiny_layer):
    # x = R^T xt with xt zero on 48 coordinates per block: the 80 screened
    # coordinates carry all of R x, so an unquantised sketch gives g^T x.
    r = _reader(tiny_layer, sketch="exact")
    rng = np.random.default_rng(21)
    rmat = rotation_matrix(r.sigma)
    for _ in range(3):
        xt = rng.choice([-1, 1], S.hidden) * rng.uniform(0.5, 2.0, S.hidden)
        zero = np.concatenate([b * 128 + rng.choice(128, 48, replace=False) for b in range(S.n_blocks)])
        xt[zero] = 0.0
        x = (rmat.T @ xt).astype(np.float32)
        _, sel = r.select(x)
        glob = (sel + 128 * np.arange(S.n_blocks)[:, None]).reshape(-1)
        assert set(glob.tolist()) == set(range(S.hidden)) - set(zero.tolist())
        ids = np.array([3, 9])
        ghat, vhat = r.screen(x, ids, sel)
        for s, e in enumerate(ids):
            g = bf16_to_f64(tiny_layer["gate"][e]) @ x.astype(np.float64)
            v = bf16_to_f64(tiny_layer["up"][e]) @ x.astype(np.float64)
            scale = np.abs(bf16_to_f64(tiny_layer["gate"][e])).sum(1) * np.abs(x).max()
            assert np.all(np.abs(ghat[s] - g) <= 1e-6 * scale)
            scale = np.abs(bf16_to_f64(tiny_layer["up"][e])).sum(1) * np.abs(x).max()
            assert np.all(np.abs(vhat[s] - v) <= 1e-6 * scale)


def test_selection_dominance(tiny_reader):
    for x in _tokens(4):
        v, sel = tiny_reader.select(x)
        for b in range(S.n_blocks):
            a = np.abs(v[b].astype(np.float64))
            ins = set(sel[b].tolist())
            outs = set(range(128)) - ins
            assert len(ins) == 80
            for i in ins:
                for j in outs:
                    assert a[i] > a[j] or (a[i] == a[j] and i < j)


def _exactly_ternary_layer(seed):
    """Rows whose rotated blocks are exactly 2^-m * 128 * c for random codes c."""
    H, E, I = 256, 4, 16
    rng = np.random.default_rng(seed)
    sig = sign_vector(777, H)
    hb = sylvester_hadamard(128)
    rows = {}
    true_alpha = {}
    for name in ("gate", "up"):
        w = np.zeros((E, I, H))
        c_all = rng.integers(-1, 2, (E, I, 2, 128))
        m_all = rng.integers(4, 9, (E, I, 2))
        for e in range(E):
            for j in range(I):
                for b in range(2):
                    c = c_all[e, j, b]
                    if not c.any():
                        c[0] = 1
                    m = m_all[e, j, b]
                    w[e, j, b * 128:(b + 1) * 128] = sig[b * 128:(b + 1) * 128] * (hb @ c) * 2.0 ** -m
        assert np.array_equal(bf16_to_f64(f32_to_bf16_bits(w.astype(np.float32))), w)
        rows[name] = f32_to_bf16_bits(w.astype(np.float32))
        true_alpha[name] = SQRT128 * 2.0 ** -m_all.astype(np.float64)  # [E][I][2]
        rows[name + "_codes"] = c_all
    down = f32_to_bf16_bits(rng.standard_normal((E, H, I)).astype(np.float32) * 0.02)
    return rows, down, true_alpha, sig


def test_ternary_screen_on_exactly_ternary_rows():
    # codes recover c exactly, alpha = fp16(sqrt(128) 2^-m), and the screen
    # equals the exact screen scaled per block by alpha16 / alpha_true.
    rows, down, ta, _ = _exactly_ternary_layer(5)
    common = dict(rank=8, n_screen=128, rot_seed=777)
    rt = OracleReader(256, 4, 16, 2, rows["gate"], rows["up"], down, **common)
    rx = OracleReader(256, 4, 16, 2, rows["gate"], rows["up"], down, sketch="exact", **common)
    for m, name in enumerate(("gate", "up")):
        c = rows[name + "_codes"]  # [E][I][2 blocks][128]
        assert np.array_equal(rt.codes[:, m], c.transpose(0, 2, 3, 1))
        g, u = unpack_units(rt.units, 16)
        assert np.array_equal((g, u)[m], rt.codes[:, m])
    x = make_tokens(workload("tiny"), 1)[0]
    ids = np.array([2, 0])
    v, sel = rt.select(x)
    gt, vt = rt.screen(x, ids, sel)
    from oracle.rotation import rotate_x_f64
    xr = rotate_x_f64(x.astype(np.float64), rt.sigma)
    for s, e in enumerate(ids):
        for m, est in enumerate((gt, vt)):
            alpha16 = rt.alpha[e, :, m, :]  # [nb][I]
            ratio = alpha16 / ta[("gate", "up")[m]][e].T  # [nb][I]
            exact_parts = np.stack([xr[b] @ rx.rot_rows[e, m, b] for b in range(2)])  # [nb][I]
            ref = (ratio * exact_parts).sum(0)
            assert np.allclose(est[s], ref, rtol=1e-12, atol=1e-14)


def _bits(a):
    return f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def test_dense_hand_worked_one_channel():
    # H = 2, one expert, one channel: g = (2, 0), v = (3, 0), d = (1, -1),
    # x = (1, 0): g.x = 2, v.x = 3, so y = 3 phi(2) (1, -1) with
    # phi(2) = 2 / (1 + e^-2).  A transposed D, a wrong activation or a
    # dropped weight gives another vector.
    gate = _bits([[[2.0, 0.0]]])          # [E][I][H]
    up = _bits([[[3.0, 0.0]]])
    down = _bits([[[1.0], [-1.0]]])       # [E][H][I]: column j is d_j
    y = dense_moe(gate, up, down, np.array([1.0, 0.0]), [0], [1.0])
    phi2 = 2.0 / (1.0 + np.exp(-2.0))
    assert np.allclose(y, [3.0 * phi2, -3.0 * phi2], rtol=1e-15, atol=0)


def test_dense_hand_worked_two_experts_weighted():
    # expert 0 as above; expert 1: g = (0, 1), v = (1, 1), d = (2, 0).
    # x = (1, -2): expert 0 has g.x = 2, v.x = 3, a = 3 phi(2); expert 1 has
    # g.x = -2, v.x = -1, a = -phi(-2) = 2 / (1 + e^2).  Weights 0.75, 0.25:
    # y = 0.75 * 3 phi(2) (1, -1) + 0.25 * 2/(1 + e^2) (2, 0).
    gate = _bits([[[2.0, 0.0]], [[0.0, 1.0]]])
    up = _bits([[[3.0, 0.0]], [[1.0, 1.0]]])
    down = _bits([[[1.0], [-1.0]], [[2.0], [0.0]]])
    x = np.array([1.0, -2.0])
    phi2 = 2.0 / (1.0 + np.exp(-2.0))
    a1 = 2.0 / (1.0 + np.exp(2.0))
    want = 0.75 * 3.0 * phi2 * np.array([1.0, -1.0]) + 0.25 * a1 * np.array([2.0, 0.0])
    y = dense_moe(gate, up, down, x, [0, 1], [0.75, 0.25])
    assert np.allclose(y, want, rtol=1e-15, atol=1e-16)
    # the routed order does not matter; an expert not routed does not count
    assert np.allclose(dense_moe(gate, up, down, x, [1, 0], [0.25, 0.75]), want, rtol=1e-15, atol=1e-16)
    assert np.allclose(dense_moe(gate, up, down, x, [0], [0.75]),
                       0.75 * 3.0 * phi2 * np.array([1.0, -1.0]), rtol=1e-15, atol=0)


def test_score_is_norm_of_channel_contribution(tiny_layer):
    # exact sketch + full screen: g_hat = g^T x, so s_j = ||w a_j d_j||_2, the
    # norm of the dense block's output with every other down column zeroed
    r = _reader(tiny_layer, sketch="exact", n_screen=128)
    x = _tokens(1)[0]
    ids, w, _ = route(tiny_layer["router"], x, S.top)
    w32 = w.astype(np.float32)
    out = r.decode(x, ids, w32, 10)
    assert (out["ghat"] < 0).any()
    for s, e in enumerate(ids):
        for j in range(S.inter):
            down = np.zeros_like(tiny_layer["down"])
            down[e, :, j] = tiny_layer["down"][e, :, j]
            contrib = dense_moe(tiny_layer["gate"], tiny_layer["up"], down, x.astype(np.float64),
                                [e], [np.float64(w32[s])])
            assert np.isclose(out["score"][s, j], np.linalg.norm(contrib), rtol=1e-6, atol=1e-12)


def test_scores_nonnegative_and_norms(tiny_reader, tiny_layer):
    x = _tokens(1)[0]
    ids, w, _ = route(tiny_layer["router"], x, S.top)
    out = tiny_reader.decode(x, ids, w, 23)
    assert (out["ghat"] < 0).any() and np.all(out["score"] >= 0)
    ref = np.linalg.norm(bf16_to_f64(tiny_layer["down"]), axis=1).astype(np.float32)
    assert np.array_equal(tiny_reader.norms, ref) or np.allclose(tiny_reader.norms, ref, rtol=2e-7)


def test_one_expert_may_take_every_kept_channel(tiny_layer, tiny_reader):
    x = _tokens(1)[0]
    ids = np.array([4, 11])
    w = np.array([0.999, 0.001], dtype=np.float32)
    out = tiny_reader.decode(x, ids, w, 23)
    assert np.all(out["kept"] < S.inter)  # all kept channels in slot 0
    assert len(out["kept"]) == 23


def test_pack_matches_codes(tiny_reader):
    g, u = unpack_units(tiny_reader.units, S.inter)
    assert np.array_equal(g, tiny_reader.codes[:, 0])
    assert np.array_equal(u, tiny_reader.codes[:, 1])
    assert tiny_reader.units.shape == (S.n_experts, S.n_blocks, 128, 32)


def test_expert_subset_build_decodes_like_the_full_build(tiny_layer, tiny_reader):
    """An oracle built for the routed experts only (load steps (1)-(2) on those,
    the recovery basis over every expert) decodes those tokens bit for bit like
    the full build, and refuses a token routed elsewhere."""
    X = _tokens(4)
    routes = [route(tiny_layer["router"], x, S.top)[:2] for x in X]
    used = sorted({int(e) for ids, _ in routes for e in ids})
    sub = _reader(tiny_layer, experts=used)
    assert np.array_equal(sub.U_bits, tiny_reader.U_bits) and np.array_equal(sub.b_bits, tiny_reader.b_bits)
    for x, (ids, w) in zip(X, routes):
        a = tiny_reader.decode(x, ids, w, 23)
        b = sub.decode(x, ids, w, 23)
        for key in ("ghat", "vhat", "score", "kept", "y"):
            assert np.array_equal(a[key], b[key]), key
    other = next(e for e in range(S.n_experts) if e not in used)
    ids = np.array([other] + list(routes[0][0][1:]))
    with pytest.raises(ValueError):
        sub.decode(X[0], ids, routes[0][1], 23)
