"""GPU parity on the method's degenerate inputs and a wider random sweep, on
the Qwen3-30B-A3B-shaped layer:
  * x = 0: every rotated value, estimate and score is zero, so the screen's
    coordinates and the kept set are decided by the tie rule alone (lower
    index first), through the top-k's general path (the boundary bin holds
    every candidate);
  * one nonzero coordinate of x;
  * all routing weight on one expert: the other slots' scores are exactly
    zero, and k beyond one expert's channels keeps zero-score channels by
    index;
  * x scaled by 1000 (the screen's fixed-point range);
  * a NaN coordinate in one token of a batch: that token's y is NaN and the
    other tokens are untouched (every index the kernels use comes from
    ranges, never from the token's values);
  * a sweep over random routings and k = 1 .. top*I - 1."""
import numpy as np
import pytest

from tests._parity import check_token

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

torch = pytest.importorskip("torch")

from calibration_free_channel_amd import Config, Reader  # noqa: E402
from oracle import OracleReader  # noqa: E402
from synth import make_layer, make_routing_inputs, make_tokens, workload  # noqa: E402

WL = workload("qwen3-30b-a3b")
S = WL.shape


@pytest.fixture(scope="module")
def c2():
    layer = make_layer(WL)
    o = OracleReader(S.hidden, S.n_experts, S.inter, S.top, layer["gate"], layer["up"], layer["down"],
                     rot_seed=WL.rot_seed)
    r = Reader.build(Config(hidden=S.hidden, n_experts=S.n_experts, inter=S.inter, top=S.top,
                            rot_seed=WL.rot_seed, max_batch=4), layer["gate"], layer["up"], layer["down"])
    yield o, r
    r.close()


def _run(o, r, X, ids, w, k):
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    lib = {n: v.cpu().numpy() for n, v in r.decode_debug(d(X), d(ids), d(w), k).items()}
    y = r.decode(d(X), d(ids), d(w), k).cpu().numpy()
    assert np.array_equal(y, lib["y"])
    for t in range(X.shape[0]):
        ref = o.decode(X[t], ids[t], w[t], k)
        check_token(lib, ref, o, X[t], ids[t], w[t], k, t)
    return lib


def _routing(n, seed):
    ids, w = make_routing_inputs(WL, n, seed_offset=seed)
    return ids.astype(np.int32), w.astype(np.float32)


@pytest.mark.parametrize("k", [1, 756, 3000])
def test_zero_token(c2, k):
    o, r = c2
    X = np.zeros((2, S.hidden), np.float32)
    ids, w = _routing(2, 31)
    lib = _run(o, r, X, ids, w, k)
    assert not lib["y"].any()
    # every score ties at zero: the kept set is the first k candidates
    assert np.array_equal(lib["kept"][0], np.arange(k))
    assert np.array_equal(lib["sel"][0], np.tile(np.arange(S.n_screen), (S.hidden // 128, 1)))


def test_one_hot_token(c2):
    o, r = c2
    X = np.zeros((2, S.hidden), np.float32)
    X[0, 5] = 3.0
    X[1, 1500] = -0.25
    ids, w = _routing(2, 32)
    _run(o, r, X, ids, w, 756)


@pytest.mark.parametrize("k", [500, 1000, 6000])
def test_all_weight_on_one_expert(c2, k):
    o, r = c2
    X = make_tokens(WL, 2, seed_offset=33)
    ids, _ = _routing(2, 33)
    w = np.zeros((2, S.top), np.float32)
    w[:, 0] = 1.0
    lib = _run(o, r, X, ids, w, k)
    if k > S.inter:
        # slot 0's channels, then the zero-score channels of slot 1 by index
        assert np.array_equal(lib["kept"][0][S.inter:], np.arange(S.inter, k))


def test_large_activations(c2):
    o, r = c2
    X = make_tokens(WL, 2, seed_offset=34) * np.float32(1000.0)
    ids, w = _routing(2, 34)
    _run(o, r, X, ids, w, 756)


def test_random_sweep(c2):
    o, r = c2
    rng = np.random.default_rng(35)
    X = make_tokens(WL, 48, seed_offset=35)
    ids, w = _routing(48, 35)
    for b0 in range(0, 48, 4):
        k = int(rng.integers(1, S.n_cand))
        sl = slice(b0, b0 + 4)
        _run(o, r, X[sl], ids[sl], w[sl], k)


@pytest.mark.parametrize("k", [1, 756])
def test_nan_token_is_isolated(c2, k):
    o, r = c2
    X = make_tokens(WL, 3, seed_offset=41)
    X[1, 5] = np.nan
    ids, w = _routing(3, 41)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    lib = {n: v.cpu().numpy() for n, v in r.decode_debug(d(X), d(ids), d(w), k).items()}
    y = r.decode(d(X), d(ids), d(w), k).cpu().numpy()
    assert np.array_equal(y, lib["y"], equal_nan=True)
    assert np.isnan(y[1]).all()
    for t in (0, 2):
        ref = o.decode(X[t], ids[t], w[t], k)
        check_token(lib, ref, o, X[t], ids[t], w[t], k, t)
    # the next call on the same reader is exact again (the accumulators
    # were cleared, whatever the NaN token left in them)
    _run(o, r, X[[0, 2]], ids[[0, 2]], w[[0, 2]], k)
