"""Seeded synthetic indexer scores (input generation only; none of the method's arithmetic).

Stand-in for a sparse-attention indexer's per-token scores (the note, section 2: the backend's
indexer picks the selected set): for request r, layer l and step t, over positions
0 .. ctx-1,
    score = importance[r, l, p] + noise * N_t[r, l, p] + (recency if p >= ctx - window),
importance and N_t independent standard normals keyed by (seed, r, l) and (seed, r, l, t), so
the top-k is the recency window plus a slowly churning set of important history positions,
and each layer selects differently.  float32.
"""
from __future__ import annotations

import numpy as np


def importance(seed: int, r: int, layer: int, ctx: int) -> np.ndarray:
    return np.random.default_rng([seed, 7, r, layer]).standard_normal(ctx, dtype=np.float32)


def step_scores(seed: int, r: int, layer: int, t: int, ctx: int, window: int, noise: float = 0.08,
                recency: float = 100.0, stride: int | None = None) -> np.ndarray:
    s = importance(seed, r, layer, ctx)
    s += np.float32(noise) * np.random.default_rng([seed, 11, r, layer, t]).standard_normal(ctx, dtype=np.float32)
    s[max(0, ctx - window):] += np.float32(recency)
    if stride is not None and stride > ctx:
        s = np.concatenate([s, np.full(stride - ctx, -np.inf, dtype=np.float32)])
    return s


def batch(seed: int, n: int, layer: int, t: int, ctx: int, window: int, stride: int, **kw) -> np.ndarray:
    return np.stack([step_scores(seed, r, layer, t, ctx, window, stride=stride, **kw) for r in range(n)])
