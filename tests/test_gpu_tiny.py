"""GPU parity on the tiny layer (hidden 256, 16 experts, intermediate 64, top-2):
the HIP library through the C ABI vs the oracle, element by element."""
import numpy as np
import pytest

from tests._parity import check_kept, check_token, rel_l2, rel_max_err

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from calibration_free_channel_amd import Config, Reader  # noqa: E402
from oracle import OracleReader, dense_moe, route  # noqa: E402
from oracle.numerics import f16_bits_to_f64  # noqa: E402
from synth import make_layer, make_tokens, workload  # noqa: E402

WL = workload("tiny")
S = WL.shape


def _cfg(**kw):
    base = dict(hidden=S.hidden, n_experts=S.n_experts, inter=S.inter, top=S.top,
                rot_seed=WL.rot_seed, max_batch=8)
    base.update(kw)
    return Config(**base)


@pytest.fixture(scope="module")
def layer():
    return make_layer(WL)


@pytest.fixture(scope="module")
def oracle(layer):
    return OracleReader(S.hidden, S.n_experts, S.inter, S.top, layer["gate"], layer["up"],
                        layer["down"], layer["router"], rot_seed=WL.rot_seed)


@pytest.fixture(scope="module")
def reader(layer):
    r = Reader.build(_cfg(), layer["gate"], layer["up"], layer["down"], layer["router"])
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
    assert np.array_equal(st["sigma"].astype(np.float64), oracle.sigma)
    # U spans the oracle's top-32 left singular space (fp16 storage)
    u = f16_bits_to_f64(st["U"])
    p_lib, p_ref = u @ u.T, oracle.U64 @ oracle.U64.T
    assert np.abs(p_lib - p_ref).max() < 5e-3
    # U b reproduces the oracle's projection of every down column
    b = f16_bits_to_f64(st["b"])
    assert rel_l2(np.einsum("hr,eir->eih", u, b), np.einsum("hr,eir->eih", oracle.U, oracle.b)) < 2e-3


@pytest.mark.parametrize("k", [23, 0, 1, 64, 127, 128])
def test_decode_parity(reader, oracle, layer, k):
    X = make_tokens(WL, 16)
    ids, w = _routed(layer, X)
    for b0 in range(0, 16, 8):
        xs, i_s, w_s = X[b0:b0 + 8], ids[b0:b0 + 8], w[b0:b0 + 8]
        lib = _np(reader.decode_debug(_dev(xs), _dev(i_s), _dev(w_s), k))
        torch.cuda.synchronize()
        for t in range(xs.shape[0]):
            ref = oracle.decode(xs[t], i_s[t], w_s[t], k)
            check_token(lib, ref, oracle, xs[t], i_s[t], w_s[t], k, t)


def test_decode_fast_path_equals_debug_path(reader, layer):
    X = make_tokens(WL, 8, seed_offset=3)
    ids, w = _routed(layer, X)
    y1 = reader.decode(_dev(X), _dev(ids), _dev(w), 23)
    d = reader.decode_debug(_dev(X), _dev(ids), _dev(w), 23)
    y2 = reader.decode(_dev(X), _dev(ids), _dev(w), 23)
    torch.cuda.synchronize()
    assert torch.equal(y1, d["y"]) and torch.equal(y1, y2), "decode is not deterministic"


def test_dense_baseline_matches_textbook_mlp(reader, layer):
    X = make_tokens(WL, 8)
    ids, w = _routed(layer, X)
    y = reader.dense(_dev(X), _dev(ids), _dev(w)).cpu().numpy()
    for t in range(8):
        ref = dense_moe(layer["gate"], layer["up"], layer["down"], X[t], ids[t], w[t])
        assert rel_l2(y[t], ref) < 1e-4


def test_keep_all_equals_dense(reader, layer):
    X = make_tokens(WL, 4)
    ids, w = _routed(layer, X)
    y = reader.decode(_dev(X), _dev(ids), _dev(w), S.n_cand).cpu().numpy()
    yd = reader.dense(_dev(X), _dev(ids), _dev(w)).cpu().numpy()
    assert rel_l2(y, yd) < 1e-5


def test_full_screen_variant(layer):
    r = Reader.build(_cfg(n_screen=128), layer["gate"], layer["up"], layer["down"])
    o = OracleReader(S.hidden, S.n_experts, S.inter, S.top, layer["gate"], layer["up"],
                     layer["down"], n_screen=128, rot_seed=WL.rot_seed)
    X = make_tokens(WL, 4)
    ids, w = _routed(layer, X)
    lib = _np(r.decode_debug(_dev(X), _dev(ids), _dev(w), 23))
    for t in range(4):
        check_token(lib, o.decode(X[t], ids[t], w[t], 23), o, X[t], ids[t], w[t], 23, t)
    r.close()


def test_out_of_range_ids_are_clamped_and_flagged(reader, layer):
    X = make_tokens(WL, 1)
    ids = np.array([[S.n_experts, 0]], dtype=np.int32)
    w = np.array([[0.6, 0.4]], dtype=np.float32)
    assert reader.status() == 0
    reader.decode(_dev(X), _dev(ids), _dev(w), 23)
    assert reader.status() == 1
    assert reader.status() == 0


def test_clone_is_identical(reader, layer):
    c = reader.clone()
    X = make_tokens(WL, 2)
    ids, w = _routed(layer, X)
    y1 = reader.decode(_dev(X), _dev(ids), _dev(w), 23)
    y2 = c.decode(_dev(X), _dev(ids), _dev(w), 23)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    c.close()


def test_argument_errors(reader):
    from calibration_free_channel_amd._lib import CfrError
    x = torch.zeros((2, S.hidden), device="cuda")
    ids = torch.zeros((2, S.top), dtype=torch.int32, device="cuda")
    w = torch.zeros((2, S.top), device="cuda")
    with pytest.raises(CfrError):
        reader.decode(x, ids, w, S.n_cand + 1)
    with pytest.raises(CfrError):
        reader.decode(x, ids, w, -1)
    with pytest.raises(ValueError):
        reader.decode(x.double(), ids, w, 3)
    big = torch.zeros((9, S.hidden), device="cuda")
    with pytest.raises(CfrError):
        reader.decode(big, torch.zeros((9, S.top), dtype=torch.int32, device="cuda"),
                      torch.zeros((9, S.top), device="cuda"), 3)


def test_stages_in_order_equal_decode(reader, layer):
    """The measurement entry (one kernel per call) run as screen, select,
    reduce reproduces cfr_reader_decode bit for bit; a bad stage is refused."""
    from calibration_free_channel_amd._lib import CfrError
    X = make_tokens(WL, 4, seed_offset=11)
    ids, w = _routed(layer, X)
    x, i, ww = _dev(X), _dev(ids), _dev(w)
    y_ref = reader.decode(x, i, ww, 23)
    y = torch.empty_like(y_ref)
    for stage in range(3):
        reader.decode_stage(stage, x, i, ww, 23, out=y)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    with pytest.raises(CfrError):
        reader.decode_stage(3, x, i, ww, 23, out=y)
