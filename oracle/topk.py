"""Exact top-k keep rule.  (Oracle: test infrastructure.)

The reader keeps exactly the k highest-scoring channels of the token across
all routed experts, so one expert may take many channels and another none
([zh §前置知识 / keep rule]; [zh §核心方法]; [ko §어떻게 쓰나]).

Reading: ties go to the lower candidate index (candidate = slot * I + j).

Pins (tests/test_oracle_topk.py): brute force over all k-subsets on tiny
inputs, and a stable full sort on random inputs with planted ties.
"""
import numpy as np


def topk_desc(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores (ties -> lower index), sorted ascending."""
    s = np.asarray(scores)
    order = np.lexsort((np.arange(s.shape[0]), -s))  # primary: -s, secondary: index
    return np.sort(order[:k])
