"""GPU parity of the batch-shared decode (cfr_reader_decode_shared) against
the oracle's batch-shared selection (oracle/shared.py): the union of routed
experts exactly; the batch scores within 2e-5 of the largest (float32 sums of
a few per-token scores against float64); the kept union candidates equal
outside a relative band of 1e-4 around the oracle's k-th batch score (the
oracle's y is then recomputed on the library's kept set); every token's y
within 2e-3 relative L2.  Tiny layer over batches 1..8 and the edge budgets,
the Qwen3-30B-A3B layer at batch 4 and the Qwen3-235B-A22B layer (128
experts) at batch 8, each at the per-token budget's share of the union."""
import sys

import numpy as np
import pytest

from tests._parity import KEPT_BAND, Y_RTOL, rel_l2, rel_max_err

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

torch = pytest.importorskip("torch")

from calibration_free_channel_amd import Config, Reader  # noqa: E402
from calibration_free_channel_amd._lib import CfrError  # noqa: E402
from oracle import OracleReader, decode_shared  # noqa: E402
from synth import make_layer, make_routing_inputs, make_tokens, workload  # noqa: E402


def _log(msg):
    print(f"[shared] {msg}", flush=True)
    sys.stdout.flush()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _check(reader, oracle, X, ids, w, k):
    lib = reader.decode_shared(_dev(X), _dev(ids), _dev(w), k, debug=True)
    lib = {n: v.cpu().numpy() for n, v in lib.items()}
    ref = decode_shared(oracle, X, ids, w, k)
    assert np.array_equal(lib["experts"], ref["experts"])
    bs = ref["bscore"].reshape(-1)
    assert rel_max_err(lib["bscore"], bs) <= 2e-5
    kk = min(k, bs.size)
    kept = lib["kept"].astype(np.int64)
    assert kept.shape == (kk,) and np.all(np.diff(kept) > 0)
    diff = set(kept.tolist()) ^ set(ref["kept"].tolist())
    if kk:
        sk = np.sort(bs)[::-1][kk - 1]
        for c in diff:
            assert abs(bs[c] - sk) <= KEPT_BAND * max(sk, 1e-30), (c, bs[c], sk)
    if diff:
        ref = decode_shared(oracle, X, ids, w, k, kept=kept)
    errs = [rel_l2(lib["y"][t], ref["y"][t]) for t in range(X.shape[0])]
    assert max(errs) <= Y_RTOL, errs
    fast = reader.decode_shared(_dev(X), _dev(ids), _dev(w), k).cpu().numpy()
    assert np.array_equal(fast, lib["y"]), "debug and fast calls differ"
    return max(errs), len(diff), ref["experts"].size


TINY = workload("tiny")
TS = TINY.shape


@pytest.fixture(scope="module")
def tiny():
    L = make_layer(TINY)
    r = Reader.build(Config(hidden=TS.hidden, n_experts=TS.n_experts, inter=TS.inter, top=TS.top,
                            rot_seed=TINY.rot_seed, max_batch=8), L["gate"], L["up"], L["down"])
    o = OracleReader(TS.hidden, TS.n_experts, TS.inter, TS.top, L["gate"], L["up"], L["down"],
                     rot_seed=TINY.rot_seed)
    yield L, r, o
    r.close()


@pytest.mark.parametrize("batch", [1, 2, 5, 8])
@pytest.mark.parametrize("share", [0.0, 0.18, 0.5, 1.0])
def test_tiny_batches(tiny, batch, share):
    L, r, o = tiny
    X = make_tokens(TINY, batch, seed_offset=batch)
    ids, w = make_routing_inputs(TINY, batch, seed_offset=batch)
    u = np.unique(ids).size
    k = int(round(share * u * TS.inter))
    err, nd, _ = _check(r, o, X, ids, w, k)
    _log(f"tiny batch {batch} union {u} k {k}: y rel L2 {err:.2e}, band swaps {nd}")


def test_tiny_batch_of_one_matches_the_per_token_decode(tiny):
    L, r, o = tiny
    X = make_tokens(TINY, 1, seed_offset=3)
    ids, w = make_routing_inputs(TINY, 1, seed_offset=3)
    ys = r.decode_shared(_dev(X), _dev(ids), _dev(w), 23).cpu().numpy()
    yd = r.decode(_dev(X), _dev(ids), _dev(w), 23).cpu().numpy()
    assert rel_l2(ys, yd) < 1e-5


def test_tiny_shared_experts_and_k_above_the_union(tiny):
    # every token routed to the same two experts: the union is those two and
    # a k beyond 2 * inter keeps them all (the dense block for every token)
    L, r, o = tiny
    X = make_tokens(TINY, 6, seed_offset=11)
    ids = np.tile(np.array([[5, 9]], dtype=np.int32), (6, 1))
    w = np.tile(np.array([[0.7, 0.3]], dtype=np.float32), (6, 1))
    _check(r, o, X, ids, w, 100)
    y = r.decode_shared(_dev(X), _dev(ids), _dev(w), 6 * TS.top * TS.inter).cpu().numpy()
    yd = r.dense(_dev(X), _dev(ids), _dev(w)).cpu().numpy()
    assert rel_l2(y, yd) < 1e-5


@pytest.mark.parametrize("k", [1, 37, 100])
def test_tiny_all_scores_tied(tiny, k):
    # x = 0: every batch score is 0, so the kept candidates are the k lowest
    # union candidates (ties to the lower index) and every y is 0
    L, r, o = tiny
    X = np.zeros((5, TS.hidden), np.float32)
    ids, w = make_routing_inputs(TINY, 5, seed_offset=5)
    _, nd, nu = _check(r, o, X, ids, w, k)
    lib = r.decode_shared(_dev(X), _dev(ids), _dev(w), k, debug=True)
    assert nd == 0
    assert np.array_equal(lib["kept"].cpu().numpy(), np.arange(min(k, nu * TS.inter)))


def test_argument_rules(tiny):
    L, r, o = tiny
    X = _dev(make_tokens(TINY, 2))
    ids, w = make_routing_inputs(TINY, 2)
    with pytest.raises(CfrError):
        r.decode_shared(X, _dev(ids), _dev(w), 2 * TS.top * TS.inter + 1)
    with pytest.raises(CfrError):
        r.decode_shared(X, _dev(ids), _dev(w), -1)


@pytest.mark.parametrize("name,batch,k_token", [("qwen3-30b-a3b", 4, 756), ("qwen3-235b-a22b", 8, 1511)])
def test_layer_shapes(name, batch, k_token):
    wl = workload(name)
    s = wl.shape
    L = make_layer(wl)
    X = make_tokens(wl, batch, seed_offset=21)
    ids, w = make_routing_inputs(wl, batch, seed_offset=21)
    u = np.unique(ids).size
    k = int(round(k_token * u / s.top))  # the per-token budget's share of the union
    r = Reader.build(Config(hidden=s.hidden, n_experts=s.n_experts, inter=s.inter, top=s.top,
                            rot_seed=wl.rot_seed, max_batch=batch), L["gate"], L["up"], L["down"])
    try:
        o = OracleReader(s.hidden, s.n_experts, s.inter, s.top, L["gate"], L["up"], L["down"],
                         rot_seed=wl.rot_seed, experts=np.unique(ids))
        err, nd, nu = _check(r, o, X, ids, w, k)
        _log(f"{name} batch {batch}: union {nu} experts, k {k}: y rel L2 {err:.2e}, band swaps {nd}")
    finally:
        r.close()
