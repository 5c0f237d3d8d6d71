"""The allocation-free decode entry point (cfr_reader_decode_noalloc) through
the C ABI: its output equals cfr_reader_decode's bit for bit (the same
kernels on the same inputs; stricter than the 2e-3 relative L2 bar), on two
calls in a row where the second is smaller (fewer tokens, another k), on
the tiny layer and on the Qwen3-30B-A3B-shaped layer, with the ordinary
entry point's calls interleaved, and calls of two readers of different
shapes interleaved (each carves the shared array differently); a call
needing more scratch than the static array holds is refused with
CFR_EUNSUPPORTED and leaves the next call correct."""
import numpy as np
import pytest

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

torch = pytest.importorskip("torch")

from calibration_free_channel_amd import Config, Reader  # noqa: E402
from calibration_free_channel_amd._lib import CFR_EUNSUPPORTED, CfrError  # noqa: E402
from oracle import route  # noqa: E402
from synth import LayerShape, make_layer, make_tokens, workload  # noqa: E402


def _inputs(layer, wl, n, seed_offset):
    X = make_tokens(wl, n, seed_offset=seed_offset)
    ids, ws = [], []
    for x in X:
        i, w, _ = route(layer["router"], x, wl.shape.top)
        ids.append(i)
        ws.append(w.astype(np.float32))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    return dev(X), dev(np.stack(ids).astype(np.int32)), dev(np.stack(ws))


@pytest.mark.parametrize("name,calls", [("tiny", [(8, 23), (3, 10)]),
                                        ("qwen3-30b-a3b", [(4, 756), (1, 445)])])
def test_noalloc_equals_decode_on_two_calls(name, calls):
    wl = workload(name)
    s = wl.shape
    layer = make_layer(wl)
    r = Reader.build(Config(hidden=s.hidden, n_experts=s.n_experts, inter=s.inter, top=s.top,
                            rot_seed=wl.rot_seed, max_batch=max(b for b, _ in calls)),
                     layer["gate"], layer["up"], layer["down"], layer["router"])
    try:
        for n, (batch, k) in enumerate(calls):
            x, i, w = _inputs(layer, wl, batch, seed_offset=40 + n)
            y_ref = r.decode(x, i, w, k)
            y = torch.full_like(y_ref, float("nan"))
            r.decode_noalloc(x, i, w, k, out=y)
            torch.cuda.synchronize()
            assert torch.equal(y, y_ref), f"call {n}: max |diff| {(y - y_ref).abs().max().item()}"
            # and again after an ordinary decode of other inputs
            x2, i2, w2 = _inputs(layer, wl, batch, seed_offset=60 + n)
            r.decode(x2, i2, w2, k)
            y.fill_(float("nan"))
            r.decode_noalloc(x, i, w, k, out=y)
            torch.cuda.synchronize()
            assert torch.equal(y, y_ref)
        assert r.status() == 0
    finally:
        r.close()


def test_noalloc_refuses_calls_beyond_its_scratch():
    # 8 routed experts x 1024 channels: 8192 candidates per token; at 64
    # tokens the screen sums alone take 8 MiB
    shape = LayerShape(hidden=128, n_experts=16, inter=1024, top=8)
    wl = workload("tiny", shape=shape)
    layer = make_layer(wl)
    r = Reader.build(Config(hidden=128, n_experts=16, inter=1024, top=8, rot_seed=wl.rot_seed, max_batch=64),
                     layer["gate"], layer["up"], layer["down"], layer["router"])
    try:
        x, i, w = _inputs(layer, wl, 64, seed_offset=3)
        y = torch.empty((64, 128), dtype=torch.float32, device="cuda")
        with pytest.raises(CfrError) as err:
            r.decode_noalloc(x, i, w, 900, out=y)
        assert err.value.code == CFR_EUNSUPPORTED
        # a call that fits still equals the ordinary decode
        y_ref = r.decode(x[:2], i[:2], w[:2], 900)
        y2 = torch.empty_like(y_ref)
        r.decode_noalloc(x[:2], i[:2], w[:2], 900, out=y2)
        torch.cuda.synchronize()
        assert torch.equal(y2, y_ref)
    finally:
        r.close()


def test_noalloc_interleaved_readers_of_different_shapes():
    # readers whose calls carve the shared array differently: a larger call's
    # screen sums cover bytes where a smaller call left partial outputs, and
    # the other way round
    built = []
    for name, mb in (("tiny", 8), ("qwen3-30b-a3b", 4)):
        wl = workload(name)
        s = wl.shape
        layer = make_layer(wl)
        built.append((wl, layer, Reader.build(Config(hidden=s.hidden, n_experts=s.n_experts, inter=s.inter,
                                                     top=s.top, rot_seed=wl.rot_seed, max_batch=mb),
                                              layer["gate"], layer["up"], layer["down"], layer["router"])))
    try:
        for n, (which, batch, k) in enumerate([(1, 4, 756), (0, 8, 23), (1, 4, 445), (0, 1, 64), (1, 2, 756),
                                               (0, 8, 0), (1, 3, 6144)]):
            wl, layer, r = built[which]
            x, i, w = _inputs(layer, wl, batch, seed_offset=80 + n)
            y_ref = r.decode(x, i, w, k)
            y = torch.full_like(y_ref, float("nan"))
            r.decode_noalloc(x, i, w, k, out=y)
            torch.cuda.synchronize()
            assert torch.equal(y, y_ref), f"call {n} ({wl.name}, batch {batch}, k {k})"
    finally:
        for _, _, r in built:
            r.close()
