"""GPU parity at the Qwen3-235B-A22B layer as configured: hidden 4096, 128
experts, intermediate 1536, top-8 (12288 candidates per token), batch 8,
k = 1511 (12.3% of the routed channels).  This is the 512-thread select path
with eight 512-wide row chunks over 4.8 GB of resident rows.  The library
builds the whole layer (every expert sketched, the rank-32 basis over all
196 608 down columns); the oracle sketches only the experts the test tokens
route to and takes its basis over every expert's down columns too."""
import sys
import time
import numpy as np
import pytest

from tests._parity import check_token

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

torch = pytest.importorskip("torch")

from calibration_free_channel_amd import Config, Reader  # noqa: E402
from oracle import OracleReader  # noqa: E402
from synth import make_layer, make_routing_inputs, make_tokens, workload  # noqa: E402

WL = workload("qwen3-235b-a22b")
S = WL.shape
K = 1511
# the tokens of each test: (seed offset, count)
TOKENS = {"parity": (0, 8), "fast": (1, 8), "dense": (2, 8)}


def _routing(name):
    off, n = TOKENS[name]
    return make_tokens(WL, n, seed_offset=off), *make_routing_inputs(WL, n, seed_offset=off)


def _log(msg):
    print(f"[qwen3-235b-shape parity] {msg}", flush=True)
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
    used = sorted({int(e) for e in _routing("parity")[1].reshape(-1)})
    o = OracleReader(S.hidden, S.n_experts, S.inter, S.top, layer["gate"], layer["up"],
                     layer["down"], rot_seed=WL.rot_seed, experts=used)
    _log(f"oracle built in {time.time() - t:.1f}s ({len(used)} routed experts sketched, "
         f"basis over all {S.n_experts})")
    return o


@pytest.fixture(scope="module")
def reader(layer):
    t = time.time()
    r = Reader.build(Config(hidden=S.hidden, n_experts=S.n_experts, inter=S.inter, top=S.top,
                            rot_seed=WL.rot_seed, max_batch=8),
                     layer["gate"], layer["up"], layer["down"])
    _log(f"library reader built in {time.time() - t:.1f}s")
    yield r
    r.close()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_batch8_parity(reader, oracle):
    X, ids, w = _routing("parity")
    lib = {k: v.cpu().numpy() for k, v in reader.decode_debug(_dev(X), _dev(ids), _dev(w), K).items()}
    for t in range(8):
        ref = oracle.decode(X[t], ids[t], w[t], K)
        err, ndiff = check_token(lib, ref, oracle, X[t], ids[t], w[t], K, t)
        _log(f"token {t}: y rel L2 {err:.2e}, kept-set swaps inside the band {ndiff}")


def test_batch8_fast_path_matches_debug(reader):
    X, ids, w = _routing("fast")
    a = reader.decode(_dev(X), _dev(ids), _dev(w), K)
    b = reader.decode_debug(_dev(X), _dev(ids), _dev(w), K)["y"]
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_dense_block_batch8(reader, layer):
    """The dense BF16 block (eight 512-wide chunks per row, one channel in
    flight per wave) against the textbook gated MLP, float64."""
    from oracle import dense_moe
    from tests._parity import rel_l2
    X, ids, w = _routing("dense")
    y = reader.dense(_dev(X), _dev(ids), _dev(w)).cpu().numpy()
    for t in (0, 3, 7):
        ref = dense_moe(layer["gate"], layer["up"], layer["down"], X[t], ids[t], w[t])
        err = rel_l2(y[t], ref)
        _log(f"dense token {t}: rel L2 {err:.2e}")
        assert err < 1e-4


def test_export_of_routed_experts_matches_oracle_pack(reader, oracle):
    """The device build over all 128 experts: sketch bytes, scales, rho and
    norms of the sketched experts bit for bit; the recovery basis spans the
    oracle's (projector within fp16 rounding) and U b_j matches on a sample
    of every-17th expert's channels."""
    from oracle.numerics import f16_bits_to_f64
    from tests._parity import rel_l2
    st = reader.export()
    ex = oracle.experts
    assert np.array_equal(st["codes"][ex], oracle.units)
    assert np.array_equal(st["scales"][ex], oracle.alpha_bits)
    assert np.array_equal(st["rho"][ex], oracle.rho_bits)
    assert np.array_equal(st["norms"][ex], oracle.norms)
    u = f16_bits_to_f64(st["U"])
    assert np.abs(u @ u.T - oracle.U64 @ oracle.U64.T).max() < 5e-3
    b = f16_bits_to_f64(st["b"])
    sample = np.arange(0, S.n_experts, 17)
    rec_lib = np.einsum("hr,eir->eih", u, b[sample])
    rec_ref = np.einsum("hr,eir->eih", oracle.U, oracle.b[sample])
    assert rel_l2(rec_lib, rec_ref) < 2e-3
