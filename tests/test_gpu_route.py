"""GPU parity of the softmax top-k router (cfr_reader_route) against the
oracle's route: logits = W_router x, softmax over all experts, the top
largest kept (ties to the lower index), renormalised.  The choice is an
argmax on floating point, so the kept experts are compared exactly only
where the oracle's logits around the top-th place are separated by more than
a relative band; the weights of agreeing picks within 1e-5."""
import numpy as np
import pytest

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

torch = pytest.importorskip("torch")

from calibration_free_channel_amd import Config, Reader  # noqa: E402
from calibration_free_channel_amd._lib import CfrError  # noqa: E402
from oracle import route  # noqa: E402
from synth import LayerShape, make_layer, make_tokens, workload  # noqa: E402

BAND = 1e-5


def _check(ids, w, router_bits, X, top):
    for t in range(X.shape[0]):
        rid, rw, logits = route(router_bits, X[t], top)
        srt = np.sort(logits)[::-1]
        gap = (srt[top - 1] - srt[top]) / max(abs(srt[top - 1]), 1e-30) if top < logits.shape[0] else 1.0
        if gap > BAND:
            assert set(ids[t].tolist()) == set(rid.tolist()), (t, ids[t], rid)
            # order by weight, descending; equal-weight neighbours may swap
            for a, b in zip(ids[t].tolist(), rid.tolist()):
                if a != b:
                    assert abs(logits[a] - logits[b]) <= BAND * abs(logits[b]), (t, a, b)
            np.testing.assert_allclose(np.sort(w[t])[::-1], np.sort(rw)[::-1], rtol=0, atol=1e-5)
        assert abs(float(w[t].sum()) - 1.0) < 1e-5
        assert np.all(np.diff(w[t]) <= 1e-7), "weights not descending"


@pytest.mark.parametrize("name,batch", [("tiny", 8), ("qwen3-30b-a3b", 4)])
def test_route_matches_oracle(name, batch):
    wl = workload(name)
    s = wl.shape
    layer = make_layer(wl)
    r = Reader.build(Config(hidden=s.hidden, n_experts=s.n_experts, inter=s.inter, top=s.top,
                            rot_seed=wl.rot_seed, max_batch=batch),
                     layer["gate"], layer["up"], layer["down"], layer["router"])
    try:
        X = make_tokens(wl, 4 * batch, seed_offset=3)
        for b0 in range(0, X.shape[0], batch):
            xs = torch.from_numpy(X[b0:b0 + batch]).cuda()
            ids, w = r.route(xs)
            _check(ids.cpu().numpy(), w.cpu().numpy(), layer["router"], X[b0:b0 + batch], s.top)
    finally:
        r.close()


@pytest.mark.parametrize("hidden,n_experts,top", [(640, 13, 13), (384, 200, 16), (4096, 128, 8), (128, 5, 1),
                                                   (128, 600, 16)])
def test_route_odd_shapes(hidden, n_experts, top):
    # experts not a multiple of a workgroup's eight, top = all experts, more
    # experts than a wave has lanes, the largest token (eight chunks per
    # lane), one chunk per lane with lanes idle, more experts than the picking
    # workgroup has threads (each thread ranks several); then batch sizes that
    # shrink and grow on the same reader (each token's arrival counter is
    # reused)
    shape = LayerShape(hidden=hidden, n_experts=n_experts, inter=64, top=top)
    wl = workload("tiny", shape=shape)
    layer = make_layer(wl)
    r = Reader.build(Config(hidden=hidden, n_experts=n_experts, inter=64, top=top, rot_seed=wl.rot_seed,
                            max_batch=6),
                     layer["gate"], layer["up"], layer["down"], layer["router"])
    try:
        X = make_tokens(wl, 16, seed_offset=5)
        b0 = 0
        for batch in (6, 1, 3, 6):
            xs = torch.from_numpy(X[b0:b0 + batch]).cuda()
            ids, w = r.route(xs)
            _check(ids.cpu().numpy(), w.cpu().numpy(), layer["router"], X[b0:b0 + batch], top)
            b0 += batch
    finally:
        r.close()


def test_route_back_to_back_calls():
    # 64 routes of different tokens queued with no host synchronisation in
    # between, each into its own output rows: a pick made from a logit left
    # by the previous call (the workgroups of a call hand their logits to the
    # last of them through device-scope atomics) would show up here
    wl = workload("qwen3-30b-a3b")
    s = wl.shape
    layer = make_layer(wl)
    r = Reader.build(Config(hidden=s.hidden, n_experts=s.n_experts, inter=s.inter, top=s.top,
                            rot_seed=wl.rot_seed, max_batch=2),
                     layer["gate"], layer["up"], layer["down"], layer["router"])
    try:
        n = 64
        X = make_tokens(wl, 2 * n, seed_offset=7)
        xs = torch.from_numpy(X).cuda()
        ids = torch.empty((2 * n, s.top), dtype=torch.int32, device="cuda")
        w = torch.empty((2 * n, s.top), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        for i in range(n):
            b = 1 + (i % 2)
            r.route(xs[2 * i:2 * i + b], ids[2 * i:2 * i + b], w[2 * i:2 * i + b])
        torch.cuda.synchronize()
        rows = [2 * i + j for i in range(n) for j in range(1 + (i % 2))]
        _check(ids.cpu().numpy()[rows], w.cpu().numpy()[rows], layer["router"], X[rows], s.top)
    finally:
        r.close()


def test_route_ties_to_lower_index():
    # router rows repeated in pairs: every logit ties with its twin's, and the
    # lower expert index of each tied pair is ranked first
    wl = workload("tiny")
    s = wl.shape
    layer = make_layer(wl)
    router = layer["router"].copy()
    router[1::2] = router[0::2]
    r = Reader.build(Config(hidden=s.hidden, n_experts=s.n_experts, inter=s.inter, top=4,
                            rot_seed=wl.rot_seed, max_batch=4),
                     layer["gate"], layer["up"], layer["down"], router)
    try:
        X = make_tokens(wl, 4, seed_offset=6)
        ids, w = r.route(torch.from_numpy(X).cuda())
        ids, w = ids.cpu().numpy(), w.cpu().numpy()
        for t in range(4):
            rid, rw, _ = route(router, X[t], 4)
            assert ids[t].tolist() == rid.tolist(), (t, ids[t], rid)
            assert ids[t][0] % 2 == 0 and ids[t][1] == ids[t][0] + 1
            np.testing.assert_allclose(w[t], rw, rtol=0, atol=1e-5)
    finally:
        r.close()


def test_route_with_prenorm_matches_oracle():
    # the router reading RMSNorm(x) (unit weights): the normalised token
    # against float64, the choice against the oracle's route of it
    wl = workload("qwen3-30b-a3b")
    s = wl.shape
    layer = make_layer(wl)
    r = Reader.build(Config(hidden=s.hidden, n_experts=s.n_experts, inter=s.inter, top=s.top,
                            rot_seed=wl.rot_seed, max_batch=4),
                     layer["gate"], layer["up"], layer["down"], layer["router"])
    try:
        X = make_tokens(wl, 4, seed_offset=4) * np.float32(3.0)
        xs = torch.from_numpy(X).cuda()
        h = torch.empty_like(xs)
        ids, w = r.route(xs, norm_out=h, norm_eps=1e-6)
        H = X.astype(np.float64)
        H = H / np.sqrt(np.mean(H * H, axis=1, keepdims=True) + 1e-6)
        np.testing.assert_allclose(h.cpu().numpy(), H, rtol=1e-5, atol=1e-6)
        _check(ids.cpu().numpy(), w.cpu().numpy(), layer["router"], H.astype(np.float32), s.top)
    finally:
        r.close()


def test_route_needs_router_weights():
    wl = workload("tiny")
    s = wl.shape
    layer = make_layer(wl)
    r = Reader.build(Config(hidden=s.hidden, n_experts=s.n_experts, inter=s.inter, top=s.top,
                            rot_seed=wl.rot_seed), layer["gate"], layer["up"], layer["down"])
    try:
        with pytest.raises(CfrError):
            r.route(torch.from_numpy(make_tokens(wl, 1)).cuda())
    finally:
        r.close()


def test_route_non_finite_token_is_flagged_and_ranks_stay_a_permutation():
    # a NaN in one token makes every logit of that token NaN; an infinite
    # coordinate makes them +-inf or NaN.  The ranks must still place each
    # expert once (distinct ids in range, every slot written), the other
    # tokens of the batch are routed as usual, and bit 1 of the status word
    # records the non-finite logits.
    wl = workload("tiny")
    s = wl.shape
    layer = make_layer(wl)
    r = Reader.build(Config(hidden=s.hidden, n_experts=s.n_experts, inter=s.inter, top=s.top,
                            rot_seed=wl.rot_seed, max_batch=4),
                     layer["gate"], layer["up"], layer["down"], layer["router"])
    try:
        assert r.status() == 0
        X = make_tokens(wl, 4, seed_offset=9)
        X[1, 5] = np.nan
        X[3, 17] = np.inf
        ids_out = torch.full((4, s.top), -7, dtype=torch.int32, device="cuda")
        ids, w = r.route(torch.from_numpy(X).cuda(), ids_out=ids_out)
        ids, w = ids.cpu().numpy(), w.cpu().numpy()
        for t in range(4):
            assert len(set(ids[t].tolist())) == s.top and ids[t].min() >= 0 and ids[t].max() < s.n_experts
        _check(ids[[0, 2]], w[[0, 2]], layer["router"], X[[0, 2]], s.top)
        # an all-NaN token: every key ties, so the lowest indices win
        assert ids[1].tolist() == list(range(s.top))
        assert r.status() & 2
        # the flag is cleared by reading it, and finite tokens do not set it
        r.route(torch.from_numpy(X[[0, 2]]).cuda())
        assert r.status() == 0
    finally:
        r.close()
