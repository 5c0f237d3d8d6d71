"""GPU parity of the reader over a 4-bit checkpoint (cfr_build_reader_q4)
against the oracle run on the dequantized weights (oracle/int4.py): the
sketch, scales, rho and norms bit for bit, the recovery basis within fp16
rounding, every decode intermediate and y within the bars of the parity
helpers, and the 4-bit dense block against the textbook gated MLP.  The
checkpoint is synthetic: each channel's rows of the BF16 layer quantised to
4 bits per group of 128 (synth.make_layer_q4)."""
import sys

import numpy as np
import pytest

from tests._parity import check_token, rel_l2

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

torch = pytest.importorskip("torch")

from calibration_free_channel_amd import Config, Reader, read_bytes  # noqa: E402
from calibration_free_channel_amd._lib import CfrError  # noqa: E402
from oracle import OracleReader, dense_moe, route  # noqa: E402
from oracle.int4 import dequant_layer  # noqa: E402
from oracle.numerics import f16_bits_to_f64  # noqa: E402
from synth import make_layer_q4, make_routing_inputs, make_tokens, workload  # noqa: E402


def _log(msg):
    print(f"[q4] {msg}", flush=True)
    sys.stdout.flush()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


TINY = workload("tiny")
TS = TINY.shape


@pytest.fixture(scope="module")
def tiny():
    L = make_layer_q4(TINY)
    gate, up, down = dequant_layer(L["rows"], TS.hidden)
    cfg = Config(hidden=TS.hidden, n_experts=TS.n_experts, inter=TS.inter, top=TS.top,
                 rot_seed=TINY.rot_seed, max_batch=4, exact_bits=4)
    r = Reader.build_q4(cfg, L["rows"], L["router"])
    o = OracleReader(TS.hidden, TS.n_experts, TS.inter, TS.top, gate, up, down, L["router"],
                     rot_seed=TINY.rot_seed)
    yield L, r, o, (gate, up, down)
    r.close()


def test_tiny_export_matches_the_oracle_pack(tiny):
    L, r, o, _ = tiny
    st = r.export()
    assert np.array_equal(st["codes"], o.units)
    assert np.array_equal(st["scales"], o.alpha_bits)
    assert np.array_equal(st["rho"], o.rho_bits)
    assert np.array_equal(st["norms"], o.norms)
    u = f16_bits_to_f64(st["U"])
    assert np.abs(u @ u.T - o.U64 @ o.U64.T).max() < 5e-3


@pytest.mark.parametrize("k", [0, 1, 23, 64, 128])
def test_tiny_decode_parity(tiny, k):
    L, r, o, _ = tiny
    X = make_tokens(TINY, 4, seed_offset=2)
    ids, w = zip(*[route(L["router"], x, TS.top)[:2] for x in X])
    ids, w = np.stack(ids).astype(np.int32), np.stack(w).astype(np.float32)
    lib = {n: v.cpu().numpy() for n, v in r.decode_debug(_dev(X), _dev(ids), _dev(w), k).items()}
    for t in range(4):
        check_token(lib, o.decode(X[t], ids[t], w[t], k), o, X[t], ids[t], w[t], k, t)


def test_tiny_dense_block(tiny):
    L, r, o, (gate, up, down) = tiny
    X = make_tokens(TINY, 4, seed_offset=3)
    ids, w = make_routing_inputs(TINY, 4, seed_offset=3)
    y = r.dense(_dev(X), _dev(ids), _dev(w)).cpu().numpy()
    for t in range(4):
        assert rel_l2(y[t], dense_moe(gate, up, down, X[t], ids[t], w[t])) < 1e-4


def test_refusals(tiny):
    L, r, o, _ = tiny
    X = _dev(make_tokens(TINY, 2))
    ids, w = make_routing_inputs(TINY, 2)
    with pytest.raises(CfrError):
        r.decode_shared(X, _dev(ids), _dev(w), 10)
    bad = L["rows"].copy()
    bad[0, 0, 0, TS.hidden // 2 + 2 * (TS.hidden // 128)] = 16  # a zero point above 15
    with pytest.raises(CfrError):
        Reader.build_q4(Config(hidden=TS.hidden, n_experts=TS.n_experts, inter=TS.inter, top=TS.top,
                               exact_bits=4), bad)


def test_qwen3_30b_layer_batch1_and_batch4():
    wl = workload("qwen3-30b-a3b")
    s = wl.shape
    L = make_layer_q4(wl)
    gate, up, down = dequant_layer(L["rows"], s.hidden)
    cfg = Config(hidden=s.hidden, n_experts=s.n_experts, inter=s.inter, top=s.top, rot_seed=wl.rot_seed,
                 max_batch=4, exact_bits=4)
    r = Reader.build_q4(cfg, L["rows"])
    try:
        X = make_tokens(wl, 4, seed_offset=5)
        ids, w = make_routing_inputs(wl, 4, seed_offset=5)
        o = OracleReader(s.hidden, s.n_experts, s.inter, s.top, gate, up, down, rot_seed=wl.rot_seed,
                         experts=np.unique(ids))
        for k in (756, 445):
            lib = {n: v.cpu().numpy() for n, v in r.decode_debug(_dev(X), _dev(ids), _dev(w), k).items()}
            for t in range(4):
                err, nd = check_token(lib, o.decode(X[t], ids[t], w[t], k), o, X[t], ids[t], w[t], k, t)
                _log(f"qwen3-30b-a3b 4-bit k={k} token {t}: y rel L2 {err:.2e}, swaps {nd}")
            one = {n: v.cpu().numpy() for n, v in r.decode_debug(_dev(X[:1]), _dev(ids[:1]), _dev(w[:1]),
                                                                   k).items()}
            check_token(one, o.decode(X[0], ids[0], w[0], k), o, X[0], ids[0], w[0], k, 0)
        yd = r.dense(_dev(X), _dev(ids), _dev(w)).cpu().numpy()
        for t in range(4):
            assert rel_l2(yd[t], dense_moe(gate, up, down, X[t], ids[t], w[t])) < 1e-4
        rb = read_bytes(cfg, 756)
        assert rb["exact"] == 756 * 3232  # 3 x 1072 bytes, in whole 32-byte sectors
        assert rb["dense"] == 8 * 3 * 768 * 1072
    finally:
        r.close()
