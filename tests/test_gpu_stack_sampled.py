"""Teacher-forced per-layer parity on the 48-layer stack (Qwen3-30B-A3B-shaped
layers with independent weights, k = 756), and the routed, residual-carrying
layer step against the oracle.

Sampled layers 0, 1, 23, 46 and 47 at decode steps 0 and 511.  Each sampled
(layer, step) is fed the same seeded residual-stream state x on both sides
(token `step` of the workload's token stream drawn with seed offset `layer`),
so a layer's comparison does not inherit the rounding drift of the layers
before it.  Per (layer, step), everything on the library side runs in its
kernels through the C ABI:

  library   h = RMSNorm(x) fused into the routing (cfr_reader_route with a
            norm output), top-8 of 128 experts and their weights, then the
            decode of h at k = 756 with x added in its last kernel
            (cfr_reader_decode_residual): x + y;
  oracle    h = RMSNorm(x) in float64 (unit weights, eps 1e-6), the softmax
            top-8 router on h, the reader's decode of h.

Checks: h within float32 rounding of the float64 norm; the routed experts
equal outside the router's tie band and their weights within 1e-5; the
decode's intermediates on the library's own h and routing within the bars
of the parity helpers (coordinates, estimates, scores, kept set, y); the
fused residual equals x + y bit for bit; and the library's x + y minus x
against the oracle's end-to-end y (its own norm and routing) within the
decode's 2e-3 relative L2."""
import sys
import time

import numpy as np
import pytest

from tests._parity import Y_RTOL, check_token, rel_l2

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

torch = pytest.importorskip("torch")

from calibration_free_channel_amd import Config, Reader  # noqa: E402
from oracle import OracleReader, route  # noqa: E402
from synth import make_layer, make_tokens, workload  # noqa: E402

WL = workload("qwen3-30b-a3b-48l")
S = WL.shape
K = 756
EPS = 1e-6
LAYERS = (0, 1, 23, 46, 47)
STEPS = (0, 511)
ROUTE_BAND = 1e-5


def _log(msg):
    print(f"[stack sampled] {msg}", flush=True)
    sys.stdout.flush()


def _state(layer, step):
    """The residual-stream state fed to `layer` at decode `step`."""
    return make_tokens(WL, max(STEPS) + 1, seed_offset=layer)[step]


def _rmsnorm64(x):
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    return x / np.sqrt(np.mean(x * x) + EPS)


@pytest.mark.parametrize("layer_idx", LAYERS)
def test_teacher_forced_layer_step(layer_idx):
    t0 = time.time()
    L = make_layer(WL, layer=layer_idx)
    hs = {s: _rmsnorm64(_state(layer_idx, s)) for s in STEPS}
    oroutes = {s: route(L["router"], hs[s].astype(np.float32), S.top) for s in STEPS}
    used = sorted({int(e) for s in STEPS for e in oroutes[s][0]})
    r = Reader.build(Config(hidden=S.hidden, n_experts=S.n_experts, inter=S.inter, top=S.top,
                            rot_seed=WL.rot_seed, max_batch=1), L["gate"], L["up"], L["down"], L["router"])
    try:
        _log(f"layer {layer_idx}: reader built, {time.time() - t0:.1f}s")
        # the library's routing may pick an expert the oracle's does not (inside
        # the tie band): the oracle sketches every expert either side routes to
        steps = {}
        for s in STEPS:
            x = _state(layer_idx, s)
            xg = torch.from_numpy(x[None].copy()).cuda()
            hg = torch.empty_like(xg)
            ids, w = r.route(xg, norm_out=hg, norm_eps=EPS)
            out = r.decode(hg, ids, w, K, residual=xg)          # x + y, fused
            y_fast = r.decode(hg, ids, w, K)                    # y alone
            dbg = {n: v.cpu().numpy() for n, v in r.decode_debug(hg, ids, w, K).items()}
            torch.cuda.synchronize()
            steps[s] = dict(x=x, h=hg.cpu().numpy()[0], ids=ids.cpu().numpy()[0], w=w.cpu().numpy()[0],
                            out=out.cpu().numpy()[0], y_fast=y_fast.cpu().numpy()[0], dbg=dbg,
                            x_plus_y=(xg + y_fast).cpu().numpy()[0])
            used = sorted(set(used) | {int(e) for e in steps[s]["ids"]})
        o = OracleReader(S.hidden, S.n_experts, S.inter, S.top, L["gate"], L["up"], L["down"], L["router"],
                         rot_seed=WL.rot_seed, experts=used)
        _log(f"layer {layer_idx}: oracle built ({len(used)} experts sketched), {time.time() - t0:.1f}s")
        for s in STEPS:
            d = steps[s]
            h64 = hs[s]
            # the fused pre-norm: within a few float32 roundings of the float64 norm
            assert np.all(np.abs(d["h"] - h64) <= 8 * 2.0 ** -24 * np.abs(h64) + 1e-12), "RMSNorm"
            # the router
            rid, rw, logits = oroutes[s]
            srt = np.sort(logits)[::-1]
            gap = (srt[S.top - 1] - srt[S.top]) / max(abs(srt[S.top - 1]), 1e-30)
            same = set(d["ids"].tolist()) == set(rid.tolist())
            if gap > ROUTE_BAND:
                assert same, (layer_idx, s, d["ids"], rid)
            if same:
                lw = dict(zip(d["ids"].tolist(), d["w"].tolist()))
                assert max(abs(lw[int(e)] - float(v)) for e, v in zip(rid, rw)) <= 1e-5
            # the decode on the library's own h and routing, every intermediate
            ref = o.decode(d["h"], d["ids"], d["w"], K)
            err, nd = check_token(d["dbg"], ref, o, d["h"], d["ids"], d["w"], K)
            # the fused residual is the separate add, bit for bit
            assert np.array_equal(d["out"], d["x_plus_y"]), "fused residual differs from x + y"
            assert np.array_equal(d["y_fast"], d["dbg"]["y"][0])
            # end to end: the library's x + y - x against the oracle's own step
            e2e = rel_l2(d["out"].astype(np.float64) - d["x"].astype(np.float64),
                         o.decode(h64.astype(np.float32), rid, rw.astype(np.float32), K)["y"]) if same else None
            _log(f"layer {layer_idx} step {s}: decode y rel L2 {err:.2e} (kept swaps {nd}), "
                 f"router gap {gap:.1e}, end-to-end {e2e if e2e is None else f'{e2e:.2e}'}")
            if e2e is not None:
                assert e2e <= Y_RTOL
    finally:
        r.close()
