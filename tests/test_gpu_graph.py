"""The decode captured in a HIP graph (as bench.py times it) gives, on every
replay, bit for bit what an eager call gives: the screen accumulators are
cleared by the reduce kernel (no memset node), and nothing in the path keeps
state between calls.  Replays are interleaved with eager decodes of other
inputs and host synchronisations."""
import numpy as np
import pytest

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

torch = pytest.importorskip("torch")

from calibration_free_channel_amd import RANK_EXPECTED_ERROR, Config, Reader  # noqa: E402
from synth import make_layer, make_routing_inputs, make_tokens, workload  # noqa: E402


@pytest.mark.parametrize("ranking", [0, RANK_EXPECTED_ERROR])
def test_graph_replays_equal_eager(ranking):
    wl = workload("qwen3-30b-a3b")
    s = wl.shape
    layer = make_layer(wl)
    cfg = Config(hidden=s.hidden, n_experts=s.n_experts, inter=s.inter, top=s.top, rot_seed=wl.rot_seed,
                 max_batch=4, n_screen=128 if ranking else s.n_screen, ranking=ranking)
    k = 1234 if ranking else 756
    r = Reader.build(cfg, layer["gate"], layer["up"], layer["down"], layer["router"])
    try:
        X = torch.from_numpy(make_tokens(wl, 4, seed_offset=21)).cuda()
        ih, wh = make_routing_inputs(wl, 4, seed_offset=21)
        ids = torch.from_numpy(ih.astype(np.int32)).cuda()
        w = torch.from_numpy(wh.astype(np.float32)).cuda()
        X2 = torch.from_numpy(make_tokens(wl, 4, seed_offset=22)).cuda()
        ref = r.decode(X, ids, w, k).clone()
        y = torch.empty_like(ref)
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            r.decode(X, ids, w, k, out=y)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            r.decode(X, ids, w, k, out=y)
        torch.cuda.synchronize()
        for rep in range(4):
            y.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y, ref), f"replay {rep} differs from the eager decode"
            other = r.decode(X2, ids, w, k)  # eager work between replays
            torch.cuda.synchronize()
            assert torch.isfinite(other).all()
        del g
    finally:
        r.close()


def test_graph_of_routed_stack_layers():
    # route (with the pre-norm) and decode with the residual of two layers in one graph
    wl = workload("qwen3-30b-a3b-48l")
    s = wl.shape
    cfg = Config(hidden=s.hidden, n_experts=s.n_experts, inter=s.inter, top=s.top, rot_seed=wl.rot_seed)
    readers = []
    for l in range(2):
        L = make_layer(wl, layer=l)
        readers.append(Reader.build(cfg, L["gate"], L["up"], L["down"], L["router"]))
    try:
        x0 = torch.from_numpy(make_tokens(wl, 1)).cuda()
        x, h = torch.empty_like(x0), torch.empty_like(x0)
        ids = torch.empty((1, s.top), dtype=torch.int32, device="cuda")
        w = torch.empty((1, s.top), dtype=torch.float32, device="cuda")

        def step():
            x.copy_(x0)
            for r in readers:
                r.route(x, ids, w, norm_out=h)
                r.decode(h, ids, w, 756, out=x, residual=x)  # x += block(h), in the decode

        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            step()
        torch.cuda.synchronize()
        ref = x.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            step()
        torch.cuda.synchronize()
        for rep in range(3):
            x.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(x, ref), f"replay {rep} differs"
        del g
    finally:
        for r in readers:
            r.close()
