"""GPU parity on the Qwen3-30B-A3B-shaped layer (hidden 2048, 128 experts,
intermediate 768, top-8: 6144 candidates per token), batch 1 as timed by
bench.py and batch 4 with per-token routing and top-k, at the 17.8% (k = 756)
and 12.8% (k = 445) read budgets; batches 2, 5 and 8 at k = 756."""
import sys
import time

import numpy as np
import pytest

from tests._parity import check_token, rel_l2

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

torch = pytest.importorskip("torch")

from calibration_free_channel_amd import Config, Reader  # noqa: E402
from oracle import OracleReader, dense_moe, route  # noqa: E402
from oracle.numerics import f16_bits_to_f64  # noqa: E402
from synth import make_layer, make_tokens, workload  # noqa: E402

WL = workload("qwen3-30b-a3b")
WL4 = workload("qwen3-30b-a3b-b4")
S = WL.shape


def _log(msg):
    print(f"[qwen3-30b parity] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def layer():
    t = time.time()
    L = make_layer(WL)
    _log(f"weights generated in {time.time() - t:.1f}s")
    return L


@pytest.fixture(scope="module")
def oracle(layer):
    t = time.time()
    o = OracleReader(S.hidden, S.n_experts, S.inter, S.top, layer["gate"], layer["up"],
                     layer["down"], layer["router"], rot_seed=WL.rot_seed)
    _log(f"oracle built in {time.time() - t:.1f}s")
    return o


@pytest.fixture(scope="module")
def reader(layer):
    t = time.time()
    r = Reader.build(Config(hidden=S.hidden, n_experts=S.n_experts, inter=S.inter, top=S.top,
                            rot_seed=WL.rot_seed, max_batch=8),
                     layer["gate"], layer["up"], layer["down"], layer["router"])
    _log(f"library reader built in {time.time() - t:.1f}s")
    yield r
    r.close()


def _routed(layer, X):
    ids, ws = [], []
    for x in X:
        i, w, _ = route(layer["router"], x, S.top)
        ids.append(i)
        ws.append(w.astype(np.float32))
    return np.stack(ids).astype(np.int32), np.stack(ws)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _np(d):
    return {k: v.cpu().numpy() for k, v in d.items()}


def test_export_matches_oracle_pack(reader, oracle):
    st = reader.export()
    assert np.array_equal(st["codes"], oracle.units)
    assert np.array_equal(st["scales"], oracle.alpha_bits)
    assert np.array_equal(st["rho"], oracle.rho_bits)
    assert np.array_equal(st["norms"], oracle.norms)
    u = f16_bits_to_f64(st["U"])
    assert np.abs(u @ u.T - oracle.U64 @ oracle.U64.T).max() < 5e-3
    b = f16_bits_to_f64(st["b"])
    sample = np.arange(0, S.n_experts, 17)
    rec_lib = np.einsum("hr,eir->eih", u, b[sample])
    rec_ref = np.einsum("hr,eir->eih", oracle.U, oracle.b[sample])
    assert rel_l2(rec_lib, rec_ref) < 2e-3


@pytest.mark.parametrize("k", [756, 445])
def test_batch1_parity(reader, oracle, layer, k):
    X = make_tokens(WL, 24)
    ids, w = _routed(layer, X)
    worst, swaps = 0.0, 0
    for t in range(X.shape[0]):
        lib = _np(reader.decode_debug(_dev(X[t:t + 1]), _dev(ids[t:t + 1]), _dev(w[t:t + 1]), k))
        ref = oracle.decode(X[t], ids[t], w[t], k)
        err, nd = check_token(lib, ref, oracle, X[t], ids[t], w[t], k)
        worst, swaps = max(worst, err), swaps + nd
    _log(f"k={k}: 24 tokens, worst y rel L2 {worst:.2e}, kept swaps inside band {swaps}")


@pytest.mark.parametrize("k", [445, 756])
def test_batch4_parity(reader, oracle, layer, k):
    X = make_tokens(WL4, 16)
    ids, w = _routed(layer, X)
    for b0 in range(0, 16, 4):
        sl = slice(b0, b0 + 4)
        lib = _np(reader.decode_debug(_dev(X[sl]), _dev(ids[sl]), _dev(w[sl]), k))
        for t in range(4):
            g = b0 + t
            ref = oracle.decode(X[g], ids[g], w[g], k)
            check_token(lib, ref, oracle, X[g], ids[g], w[g], k, t)


@pytest.mark.parametrize("batch", [2, 5, 8])
def test_other_batch_sizes(reader, oracle, layer, batch):
    # the screen's block groups by batch at this layer: 1 block per
    # workgroup at batch 2, 2 at batch 5, 4 at batch 8 (512 workgroups)
    X = make_tokens(WL4, batch, seed_offset=20 + batch)
    ids, w = _routed(layer, X)
    lib = _np(reader.decode_debug(_dev(X), _dev(ids), _dev(w), 756))
    y_fast = reader.decode(_dev(X), _dev(ids), _dev(w), 756).cpu().numpy()
    assert np.array_equal(y_fast, lib["y"]), "fast path differs from the debug path"
    for t in range(batch):
        ref = oracle.decode(X[t], ids[t], w[t], 756)
        check_token(lib, ref, oracle, X[t], ids[t], w[t], 756, t)


def test_batch1_fast_path_matches_debug(reader, layer):
    X = make_tokens(WL, 4, seed_offset=9)
    ids, w = _routed(layer, X)
    for t in range(4):
        a = reader.decode(_dev(X[t:t + 1]), _dev(ids[t:t + 1]), _dev(w[t:t + 1]), 756)
        b = reader.decode_debug(_dev(X[t:t + 1]), _dev(ids[t:t + 1]), _dev(w[t:t + 1]), 756)["y"]
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def test_dense_baseline(reader, layer):
    X = make_tokens(WL, 4)
    ids, w = _routed(layer, X)
    y = reader.dense(_dev(X), _dev(ids), _dev(w)).cpu().numpy()
    for t in range(4):
        ref = dense_moe(layer["gate"], layer["up"], layer["down"], X[t], ids[t], w[t])
        assert rel_l2(y[t], ref) < 1e-4
