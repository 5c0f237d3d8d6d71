"""The library's distinct-sector count for batched calls (cfr_read_bytes_batch):
one token's call touches exactly the per-token counted reads, identical
tokens add nothing, disjoint experts add their full share, and a channel kept
by one token and skipped by another is charged both its exact rows and its b
row ([zh §前置知识 / 显存带宽受限的解码]: each touched 32-byte sector is
charged once)."""
import numpy as np
import pytest

from calibration_free_channel_amd import Config, read_bytes, read_bytes_batch
from calibration_free_channel_amd._lib import CfrError

CFG = Config(hidden=2048, n_experts=128, inter=768, top=8)


def _token(rng, experts, k):
    ids = np.sort(rng.choice(experts, 8, replace=False)).astype(np.int32)
    sel = np.stack([np.sort(rng.choice(128, 80, replace=False)) for _ in range(16)]).astype(np.uint8)
    kept = np.sort(rng.choice(6144, k, replace=False)).astype(np.int32)
    return ids, sel, kept


def test_one_token_equals_counted_reads():
    rng = np.random.default_rng(0)
    for k in (0, 1, 445, 756, 6144):
        ids, sel, kept = _token(rng, 128, k)
        got = read_bytes_batch(CFG, ids[None], sel[None], kept[None], k)
        want = read_bytes(CFG, k)
        assert got == want


def test_duplicates_and_disjoint_tokens():
    rng = np.random.default_rng(1)
    ids, sel, kept = _token(rng, 64, 756)
    one = read_bytes_batch(CFG, ids[None], sel[None], kept[None], 756)["total"]
    two = read_bytes_batch(CFG, np.stack([ids, ids]), np.stack([sel, sel]), np.stack([kept, kept]), 756)
    assert two["total"] == one
    other = ids + 64  # disjoint experts: everything but U is counted again
    both = read_bytes_batch(CFG, np.stack([ids, other]), np.stack([sel, sel]), np.stack([kept, kept]), 756)
    assert both["total"] == 2 * one - 2048 * 32 * 2
    assert both["dense"] == 2 * read_bytes(CFG, 756)["dense"]


def test_shared_expert_kept_by_one_token_skipped_by_other():
    # two tokens route the same experts with the same coordinates; token 0
    # keeps candidate 5 only, token 1 keeps candidate 6 only: candidates 5
    # and 6 are read exactly once each and their b rows once each (each is
    # skipped by the other token), every other channel's b row once
    rng = np.random.default_rng(2)
    ids, sel, _ = _token(rng, 128, 0)
    kept = np.array([[5], [6]], dtype=np.int32)
    got = read_bytes_batch(CFG, np.stack([ids, ids]), np.stack([sel, sel]), kept, 1)
    one = read_bytes(CFG, 1)
    assert got["codes"] == one["codes"] and got["scales"] == one["scales"] and got["norms"] == one["norms"]
    assert got["exact"] == 2 * 3 * 2048 * 2
    assert got["b"] == 6144 * 32 * 2


def test_screened_coordinates_union():
    # a second token with disjoint coordinates on the same experts doubles
    # the code bytes (80 + 48 of 128 coordinates are distinct at most)
    rng = np.random.default_rng(3)
    ids, sel, kept = _token(rng, 128, 10)
    comp = np.stack([np.setdiff1d(np.arange(128), s)[:48] for s in sel]).astype(np.uint8)
    sel2 = np.concatenate([comp, np.tile(np.arange(32, dtype=np.uint8), (16, 1))], axis=1)
    sel2 = np.sort(sel2[:, :80], axis=1)
    got = read_bytes_batch(CFG, np.stack([ids, ids]), np.stack([sel, sel2]), np.stack([kept, kept]), 10)
    union = sum(len(set(a.tolist()) | set(b.tolist())) for a, b in zip(sel, sel2))
    assert got["codes"] == 8 * union * 320


def test_rejects_out_of_range():
    rng = np.random.default_rng(4)
    ids, sel, kept = _token(rng, 128, 3)
    bad = ids.copy()
    bad[0] = 128
    with pytest.raises(CfrError):
        read_bytes_batch(CFG, bad[None], sel[None], kept[None], 3)
    bad = sel.copy()
    bad[0, 0] = 200
    with pytest.raises(CfrError):
        read_bytes_batch(CFG, ids[None], bad[None], kept[None], 3)
    bad = kept.copy()
    bad[0] = 6144
    with pytest.raises(CfrError):
        read_bytes_batch(CFG, ids[None], sel[None], bad[None], 3)


def test_shared_accounting_counts_the_union_once():
    """The batch-shared count: sketch, scales and norms of the distinct
    experts at the coordinates any token screened, n_kept exact rows and the
    rest of the union's b rows, each once, and U once."""
    from calibration_free_channel_amd import read_bytes_shared
    B, nblk = 3, 16
    ids = np.array([[0, 1, 2, 3, 4, 5, 6, 7], [4, 5, 6, 7, 8, 9, 10, 11], [0, 1, 2, 3, 8, 9, 10, 11]],
                   dtype=np.int32)
    u = 12
    sel = np.tile(np.arange(80, dtype=np.uint8), (B, nblk, 1))  # every token screens the same 80
    for n_kept in (0, 5, 756, u * 768):
        st = read_bytes_shared(CFG, ids, sel, n_kept)
        assert st["codes"] == u * nblk * 80 * 320
        assert st["scales"] == u * nblk * 2 * 768 * 2
        assert st["norms"] == u * 768 * 4
        assert st["exact"] == n_kept * 3 * 2048 * 2
        assert st["b"] == (u * 768 - n_kept) * 32 * 2
        assert st["u"] == 2048 * 32 * 2
        assert st["dense"] == u * 3 * 768 * 2048 * 2
    # one token: the per-token count at k = n_kept
    one = read_bytes_shared(CFG, ids[:1], sel[:1], 756)
    assert one == read_bytes(CFG, 756)
    # a second token screening other coordinates adds their units only
    sel2 = sel.copy()
    sel2[1] = np.arange(48, 128, dtype=np.uint8)
    st = read_bytes_shared(CFG, ids[:2], sel2[:2], 0)
    # experts 0-3 and 8-11: one token each; 4-7: both, the union of 0..79 and 48..127
    assert st["codes"] == (4 * 80 + 4 * 128 + 4 * 80) * nblk * 320
    with pytest.raises(CfrError):
        read_bytes_shared(CFG, ids, sel, u * 768 + 1)
