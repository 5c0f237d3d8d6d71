"""GPU parity at edge shapes: every select geometry (2..32 candidates per
thread), every hidden-chunk count of the gather (with 8 chunks, up to two
channels per wave, one after the other), one and an odd number of
128-blocks, intermediate sizes that leave a ragged last code byte or are not
a multiple of 128, top = 1 and the largest top * inter, rank 0 (no recovery),
a rank that is not a power of two and the largest rank, partial screens of
1 and of odd sizes, k = 0, 1, ragged and all.  The HIP library through the C
ABI against the oracle, element by element, on synthetic layers of the
method's recipe (N(0, 0.02) BF16 weights with outlier input columns, x with
outlier dimensions) at these shapes."""
import numpy as np
import pytest

from tests._parity import check_token

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

torch = pytest.importorskip("torch")

from calibration_free_channel_amd import Config, Reader  # noqa: E402
from oracle import OracleReader  # noqa: E402
from synth import LayerShape, make_layer, make_routing_inputs, make_tokens, workload  # noqa: E402

# (hidden, experts, inter, top, rank, n_screen, ks); comments: what it covers
CASES = [
    (128, 4, 40, 1, 0, 1, (0, 1, 5, 40)),            # one block, top 1, rank 0, one screened coord
    (1024, 8, 333, 4, 8, 64, (0, 200, 1331, 1332)),  # 2 hidden chunks, ragged byte, 4 per thread
    (384, 16, 250, 16, 16, 128, (1, 600)),           # 3 blocks, top 16, whole sketch, 8 per thread
    (512, 32, 1024, 16, 64, 100, (2000, 16384)),     # largest top*inter (32 per thread), rank 64
    (640, 8, 96, 8, 24, 77, (3, 100, 767)),          # 5 blocks, rank 24, odd screen
    (256, 8, 640, 4, 32, 80, (300,)),                # 6 per thread
    (256, 8, 1000, 8, 32, 80, (1234,)),              # 16 per thread
    (4096, 8, 200, 4, 32, 80, (0, 7, 650, 800)),     # 8 hidden chunks, 2 channels a wave in turn
]


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _np(d):
    return {k: v.cpu().numpy() for k, v in d.items()}


@pytest.mark.parametrize("case", CASES, ids=lambda c: "H{}-E{}-I{}-top{}-r{}-ns{}".format(*c[:6]))
def test_edge_shape_parity(case):
    H, E, I, top, rank, ns, ks = case
    wl = workload("tiny", shape=LayerShape(hidden=H, n_experts=E, inter=I, top=top, rank=rank,
                                           n_screen=ns), weight_seed=7 + H + I, token_seed=11 + E)
    layer = make_layer(wl)
    o = OracleReader(H, E, I, top, layer["gate"], layer["up"], layer["down"], rank=rank,
                     n_screen=ns, rot_seed=wl.rot_seed)
    r = Reader.build(Config(hidden=H, n_experts=E, inter=I, top=top, rank=rank, n_screen=ns,
                            max_batch=3, rot_seed=wl.rot_seed),
                     layer["gate"], layer["up"], layer["down"])
    try:
        X = make_tokens(wl, 3)
        ids, w = make_routing_inputs(wl, 3)
        ids = ids.astype(np.int32)
        w = w.astype(np.float32)
        for k in ks:
            lib = _np(r.decode_debug(_dev(X), _dev(ids), _dev(w), k))
            y_fast = r.decode(_dev(X), _dev(ids), _dev(w), k).cpu().numpy()
            assert np.array_equal(y_fast, lib["y"]), "fast path differs from the debug path"
            for t in range(3):
                ref = o.decode(X[t], ids[t], w[t], k)
                check_token(lib, ref, o, X[t], ids[t], w[t], k, t)
    finally:
        r.close()
