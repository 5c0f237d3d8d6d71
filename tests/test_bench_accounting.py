"""The bench's distinct-sector count for batched calls (union_bytes): one
token's call touches exactly the per-token counted reads of the library's
accounting, identical tokens add nothing, and disjoint experts add their full
share."""
import numpy as np

import bench
from calibration_free_channel_amd import Config, read_bytes


def _token(rng, experts, k):
    ids = np.sort(rng.choice(experts, 8, replace=False))
    sel = np.stack([np.sort(rng.choice(128, 80, replace=False)) for _ in range(16)])
    kept = np.sort(rng.choice(6144, k, replace=False))
    return ids, sel, kept


def test_union_bytes_one_token_equals_counted_reads():
    cfg = Config(hidden=2048, n_experts=128, inter=768, top=8)
    rng = np.random.default_rng(0)
    for k in (0, 445, 756, 6144):
        ids, sel, kept = _token(rng, 128, k)
        got = bench.union_bytes(cfg, ids[None], sel[None], kept[None], k)
        assert got == read_bytes(cfg, k)["total"]


def test_union_bytes_duplicates_and_disjoint_tokens():
    cfg = Config(hidden=2048, n_experts=128, inter=768, top=8)
    rng = np.random.default_rng(1)
    ids, sel, kept = _token(rng, 64, 756)
    one = bench.union_bytes(cfg, ids[None], sel[None], kept[None], 756)
    two = bench.union_bytes(cfg, np.stack([ids, ids]), np.stack([sel, sel]), np.stack([kept, kept]), 756)
    assert two == one
    other = ids + 64  # disjoint experts: everything but U is counted again
    both = bench.union_bytes(cfg, np.stack([ids, other]), np.stack([sel, sel]), np.stack([kept, kept]), 756)
    assert both == 2 * one - 2048 * 32 * 2
