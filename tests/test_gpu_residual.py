"""The decode with the residual added in its last kernel
(cfr_reader_decode_residual, cfr_dense_decode_residual) equals the decode
followed by a separate float32 add, bit for bit: both add the same two
float32 values once.  In place (the residual is the output) and out of place,
batch 1 and 4, reader and dense block, on the Qwen3-30B-A3B-shaped layer."""
import numpy as np
import pytest

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

torch = pytest.importorskip("torch")

from calibration_free_channel_amd import Config, Reader  # noqa: E402
from calibration_free_channel_amd._lib import CfrError  # noqa: E402
from synth import make_layer, make_routing_inputs, make_tokens, workload  # noqa: E402

WL = workload("qwen3-30b-a3b")
S = WL.shape


@pytest.fixture(scope="module")
def reader():
    layer = make_layer(WL)
    r = Reader.build(Config(hidden=S.hidden, n_experts=S.n_experts, inter=S.inter, top=S.top,
                            rot_seed=WL.rot_seed, max_batch=4), layer["gate"], layer["up"], layer["down"])
    yield r
    r.close()


def _inputs(batch, seed):
    X = torch.from_numpy(make_tokens(WL, batch, seed_offset=seed)).cuda()
    ih, wh = make_routing_inputs(WL, batch, seed_offset=seed)
    ids = torch.from_numpy(ih.astype(np.int32)).cuda()
    w = torch.from_numpy(wh.astype(np.float32)).cuda()
    R = torch.from_numpy(make_tokens(WL, batch, seed_offset=seed + 50) * np.float32(7.0)).cuda()
    return X, ids, w, R


@pytest.mark.parametrize("batch", [1, 4])
@pytest.mark.parametrize("k", [0, 756, S.top * S.inter])
def test_reader_residual_equals_separate_add(reader, batch, k):
    X, ids, w, R = _inputs(batch, 40 + batch)
    ref = reader.decode(X, ids, w, k) + R
    y = reader.decode(X, ids, w, k, residual=R)
    assert torch.equal(y, ref)
    x_stream = R.clone()
    reader.decode(X, ids, w, k, out=x_stream, residual=x_stream)  # in place
    assert torch.equal(x_stream, ref)


@pytest.mark.parametrize("batch", [1, 4])
def test_dense_residual_equals_separate_add(reader, batch):
    X, ids, w, R = _inputs(batch, 60 + batch)
    ref = reader.dense(X, ids, w) + R
    assert torch.equal(reader.dense(X, ids, w, residual=R), ref)
    x_stream = R.clone()
    reader.dense(X, ids, w, out=x_stream, residual=x_stream)
    assert torch.equal(x_stream, ref)


def test_residual_must_not_be_the_input(reader):
    X, ids, w, _ = _inputs(1, 70)
    with pytest.raises(CfrError):
        reader.decode(X, ids, w, 756, residual=X)
    with pytest.raises(CfrError):
        reader.dense(X, ids, w, residual=X)
