"""Top-k selection from indexer scores -- TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The step before the resolver (the HiSparse note, section 2: the backend's indexer decides
which KV entries a step selects; paper abstract: the method is indexer-agnostic).  Plain
definition: for each request, among positions 0 .. len-1, the k positions of largest score,
a tie going to the smaller position, listed in ascending position order; when len < k every
position is selected and the rest of the row is -1.  Scores are finite or -inf (no NaN).

Written out with a stable sort; pinned in tests/test_oracle_topk_pins.py by brute force over
all k-subsets, closed forms and the order invariant.
"""
from __future__ import annotations

import numpy as np


def topk(scores: np.ndarray, lens: np.ndarray, k: int) -> np.ndarray:
    """scores float32 [n][>= max len], lens int [n] -> int32 [n][k]."""
    n = scores.shape[0]
    out = np.full((n, k), -1, dtype=np.int32)
    for r in range(n):
        L = int(lens[r])
        s = np.asarray(scores[r, :L], dtype=np.float64)    # exact: float32 values widen losslessly
        # descending score, ascending position: a stable sort on -score keeps positions in order
        order = np.argsort(-s, kind="stable")
        pick = np.sort(order[:k])
        out[r, : pick.size] = pick
    return out
