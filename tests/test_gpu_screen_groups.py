"""GPU parity of the screen's block groups: at batch >= 2 (score ranking,
n_screen <= 80) one screen workgroup covers 2, 4 or 8 consecutive 128-blocks
of a (token, slot, half), whatever group leaves at least 512 workgroups, and
sums them before its atomics.  These shapes reach every (words-per-thread
group, blocks-per-group) pair the library launches, with groups cut short by
the block count, against the oracle element by element (estimates, scores,
kept set, y) for every token of the batch.

(ng: threads per code word, from ceil(inter / 20) words per half; bg: blocks
per group.)"""
import numpy as np
import pytest

from tests._parity import check_token

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

torch = pytest.importorskip("torch")

from calibration_free_channel_amd import Config, Reader  # noqa: E402
from oracle import OracleReader  # noqa: E402
from synth import LayerShape, make_layer, make_routing_inputs, make_tokens, workload  # noqa: E402

# (hidden, experts, inter, top, batch, n_screen, ks); comment: ng, bg, groups
CASES = [
    (2048, 16, 100, 4, 8, 80, (0, 400)),         # ng 16, bg 2, 16 blocks
    (2048, 16, 100, 8, 8, 80, (0, 300, 800)),    # ng 16, bg 4, 16 blocks
    (1280, 32, 100, 16, 8, 80, (1, 640)),        # ng 16, bg 8, 10 blocks: a group of 2
    (1152, 16, 700, 8, 8, 77, (500, 5600)),      # ng 8, bg 2, 9 blocks: a group of 1
    (2048, 32, 700, 16, 4, 80, (1500,)),         # ng 8, bg 4, 16 blocks
    (1152, 32, 700, 16, 8, 80, (2000,)),         # ng 8, bg 8, 9 blocks: a group of 1
    (1152, 16, 1300, 8, 8, 80, (1000,)),         # ng 4, bg 2, 9 blocks: a group of 1
    (2048, 16, 1300, 8, 8, 64, (1800,)),         # ng 4, bg 4, 16 blocks, 64 screened
]


def _plan(H, I, top, B, ns):
    """The (ng, bg) the library's planner picks (for the test ids)."""
    nd = -(-I // 20)
    ng = 16
    while ng > 1 and ng * nd > 512:
        ng //= 2
    nblk = H // 128
    bg = 1
    if B >= 2 and ng >= 4 and ns <= ng * {16: 5, 8: 10, 4: 20}[ng]:
        while bg < 8 and B * top * 2 * (-(-nblk // (2 * bg))) >= 512:
            bg *= 2
    return ng, bg


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "H{}-E{}-I{}-top{}-b{}-ns{}".format(*c[:6])
                         + "-ng{}-bg{}".format(*_plan(c[0], c[2], c[3], c[4], c[5])))
def test_screen_group_parity(case):
    H, E, I, top, B, ns, ks = case
    assert _plan(H, I, top, B, ns)[1] > 1
    wl = workload("tiny", shape=LayerShape(hidden=H, n_experts=E, inter=I, top=top, rank=16,
                                           n_screen=ns), weight_seed=3 + H + I, token_seed=5 + E)
    layer = make_layer(wl)
    o = OracleReader(H, E, I, top, layer["gate"], layer["up"], layer["down"], rank=16,
                     n_screen=ns, rot_seed=wl.rot_seed)
    r = Reader.build(Config(hidden=H, n_experts=E, inter=I, top=top, rank=16, n_screen=ns,
                            max_batch=B, rot_seed=wl.rot_seed),
                     layer["gate"], layer["up"], layer["down"])
    try:
        X = make_tokens(wl, B)
        ids, w = make_routing_inputs(wl, B)
        ids = ids.astype(np.int32)
        w = w.astype(np.float32)
        for k in ks:
            lib = {n: v.cpu().numpy() for n, v in r.decode_debug(_dev(X), _dev(ids), _dev(w), k).items()}
            y_fast = r.decode(_dev(X), _dev(ids), _dev(w), k).cpu().numpy()
            assert np.array_equal(y_fast, lib["y"]), "fast path differs from the debug path"
            for t in range(B):
                ref = o.decode(X[t], ids[t], w[t], k)
                check_token(lib, ref, o, X[t], ids[t], w[t], k, t)
    finally:
        r.close()
