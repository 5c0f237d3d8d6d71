"""Pins for the exact top-k keep rule: brute force over all subsets."""
import itertools

import numpy as np

from oracle.topk import topk_desc


def _dominates(s, a, b):
    return s[a] > s[b] or (s[a] == s[b] and a < b)


def test_topk_brute_force_all_subsets():
    rng = np.random.default_rng(11)
    for trial in range(400):
        n = int(rng.integers(1, 9))
        s = rng.integers(0, 4, n).astype(np.float64)  # many ties
        if trial % 2:
            s = rng.random(n)
        for k in range(n + 1):
            valid = [set(c) for c in itertools.combinations(range(n), k)
                     if all(_dominates(s, a, b) for a in c for b in set(range(n)) - set(c))]
            assert len(valid) == 1
            assert set(topk_desc(s, k).tolist()) == valid[0]


def test_topk_matches_stable_sort_with_ties():
    rng = np.random.default_rng(12)
    s = np.round(rng.random(6144), 3)  # planted ties
    for k in (0, 1, 445, 756, 6144):
        got = topk_desc(s, k)
        ref = np.sort(sorted(range(6144), key=lambda i: (-s[i], i))[:k])
        assert np.array_equal(got, ref)
        assert np.all(np.diff(got) > 0)
