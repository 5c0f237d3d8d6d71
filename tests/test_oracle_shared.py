"""Pins of the batch-shared selection oracle (oracle/shared.py) against what
the per-token method and the mathematics fix."""
import itertools

import numpy as np
import pytest

from oracle import OracleReader, decode_shared, dense_moe, route
from synth import LayerShape, make_layer, make_tokens, workload

TINY = workload("tiny")
S = TINY.shape


@pytest.fixture(scope="module")
def layer():
    return make_layer(TINY)


@pytest.fixture(scope="module")
def oracle(layer):
    return OracleReader(S.hidden, S.n_experts, S.inter, S.top, layer["gate"], layer["up"],
                        layer["down"], layer["router"], rot_seed=TINY.rot_seed)


def _routed(layer, X):
    r = [route(layer["router"], x, S.top)[:2] for x in X]
    return np.stack([a for a, _ in r]).astype(np.int32), np.stack([b for _, b in r]).astype(np.float32)


def _to_union(ids, kept_tok, experts):
    """Per-token candidates (slot * I + j) as union candidates (u * I + j)."""
    u = {int(e): i for i, e in enumerate(experts.tolist())}
    return np.sort([u[int(ids[c // S.inter])] * S.inter + c % S.inter for c in kept_tok])


@pytest.mark.parametrize("k", [0, 1, 23, 64, 128])
def test_batch_of_one_is_the_per_token_decode(layer, oracle, k):
    X = make_tokens(TINY, 3)
    ids, w = _routed(layer, X)
    for t in range(3):
        sh = decode_shared(oracle, X[t:t + 1], ids[t:t + 1], w[t:t + 1], k)
        ref = oracle.decode(X[t], ids[t], w[t], k)
        assert np.array_equal(sh["kept"], _to_union(ids[t], ref["kept"], sh["experts"]))
        np.testing.assert_allclose(sh["y"][0], ref["y"], rtol=1e-12, atol=1e-14 * np.abs(ref["y"]).max())


def test_two_copies_keep_the_per_token_set(layer, oracle):
    X = make_tokens(TINY, 2)
    ids, w = _routed(layer, X)
    X2 = np.stack([X[0], X[0]])
    sh = decode_shared(oracle, X2, np.stack([ids[0], ids[0]]), np.stack([w[0], w[0]]), 23)
    ref = oracle.decode(X[0], ids[0], w[0], 23)
    # the batch scores are twice the token's (exact in binary), so the order
    # and the kept set are the token's
    assert np.array_equal(sh["kept"], _to_union(ids[0], ref["kept"], sh["experts"]))
    for t in range(2):
        np.testing.assert_allclose(sh["y"][t], ref["y"], rtol=1e-12, atol=1e-14 * np.abs(ref["y"]).max())


def test_keep_every_union_candidate_is_the_dense_block(layer, oracle):
    X = make_tokens(TINY, 4)
    ids, w = _routed(layer, X)
    n_union = np.unique(ids).size * S.inter
    sh = decode_shared(oracle, X, ids, w, n_union)
    assert sh["kept"].size == n_union
    for t in range(4):
        ref = dense_moe(layer["gate"], layer["up"], layer["down"], X[t], ids[t], w[t])
        np.testing.assert_allclose(sh["y"][t], ref, rtol=1e-12, atol=1e-13 * np.abs(ref).max())
        assert np.all(sh["y_rec"][t] == 0)


def test_keep_none_is_each_tokens_recovery(layer, oracle):
    X = make_tokens(TINY, 4)
    ids, w = _routed(layer, X)
    sh = decode_shared(oracle, X, ids, w, 0)
    for t in range(4):
        ref = oracle.decode(X[t], ids[t], w[t], 0)
        assert np.all(sh["y_exact"][t] == 0)
        np.testing.assert_allclose(sh["y"][t], ref["y"], rtol=1e-12, atol=1e-14 * np.abs(ref["y"]).max())


def test_shared_rows_serve_every_token_routed_to_them(layer, oracle):
    # two tokens, one common expert: a kept channel of that expert is exact
    # for both tokens; the batch score adds the two tokens' scores
    X = make_tokens(TINY, 2, seed_offset=9)
    ids = np.array([[3, 7], [7, 11]], dtype=np.int32)
    w = np.array([[0.6, 0.4], [0.7, 0.3]], dtype=np.float32)
    sh = decode_shared(oracle, X, ids, w, 40)
    assert sh["experts"].tolist() == [3, 7, 11]
    r0 = oracle.decode(X[0], ids[0], w[0], 0)
    r1 = oracle.decode(X[1], ids[1], w[1], 0)
    d7 = oracle.norms[oracle.ix([7])[0]].astype(np.float64)
    w64 = w.astype(np.float64)  # the float32 weights the oracle reads
    s7 = w64[0, 1] * d7 * np.abs(r0["p"][1]) + w64[1, 0] * d7 * np.abs(r1["p"][0])
    np.testing.assert_allclose(sh["bscore"][1], s7, rtol=1e-15)
    # y of each token: exact on the kept channels of its experts, recovery
    # on the rest, the rows of expert 7 shared
    for t in range(2):
        kept_tok = []
        for s, e in enumerate(ids[t].tolist()):
            u = sh["experts"].tolist().index(e)
            kept_tok += [s * S.inter + (c - u * S.inter) for c in sh["kept"] if c // S.inter == u]
        ref = oracle.decode(X[t], ids[t], w[t], len(kept_tok), kept=np.array(kept_tok, dtype=np.int64))
        np.testing.assert_allclose(sh["y"][t], ref["y"], rtol=1e-12, atol=1e-14 * np.abs(ref["y"]).max())


def test_kept_set_maximises_the_summed_batch_score_brute_force():
    # a layer small enough to try every k-subset of the union candidates
    shape = LayerShape(hidden=128, n_experts=4, inter=3, top=2)
    wl = workload("tiny", shape=shape)
    L = make_layer(wl)
    o = OracleReader(128, 4, 3, 2, L["gate"], L["up"], L["down"], rank=8, rot_seed=wl.rot_seed)
    X = make_tokens(wl, 3)
    ids = np.array([[0, 1], [1, 2], [2, 3]], dtype=np.int32)
    w = np.array([[0.5, 0.5], [0.8, 0.2], [0.3, 0.7]], dtype=np.float32)
    for k in (1, 4, 7):
        sh = decode_shared(o, X, ids, w, k)
        flat = sh["bscore"].reshape(-1)
        best = max(itertools.combinations(range(flat.size), k), key=lambda c: (sum(flat[list(c)]), [-i for i in c]))
        assert sh["kept"].tolist() == sorted(best)
