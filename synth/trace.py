"""Seeded synthetic top-k selection traces (input generator only).

A decode-time indexer picks, per request and step, k token positions out of the
context.  With the indexer's weights out of reach, a trace here is built from
two parts whose mix follows the workloads the HiSparse pages describe (top-k
2048 selections over 32k-128k contexts, with a device buffer of 2048-6144 slots
that misses less as it grows, "HiSparse: Hierarchical Memory for Sparse
Attention" note, section 3 and Fig. 3):

* a recency window: the last ``window`` positions of the current context;
* a history set of ``k - window`` distinct older positions, drawn from a Zipf(s)
  popularity law over a per-request random ranking of positions (popularity is
  not tied to distance), of which a fraction ``churn`` is dropped and redrawn at
  each step.

With pages (the NSA and Quest families of the paper abstract select blocks of
consecutive tokens) the same recipe runs over page indices: ``grow_per`` tokens
per page, so a context growing by a token per step gains a page every
``grow_per`` steps and its newest page is partly written in between.

The set is emitted in a shuffled order on purpose: consumers must not rely on
sorted input.  Everything is seeded from (seed, request), so a trace is the
same on every machine and for every buffer size of a sweep.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class TraceSpec:
    n: int            # requests
    k: int            # selections per step
    ctx: int          # context length at step 0
    window: int       # recency window length
    zipf_s: float     # Zipf exponent of the history popularity law
    churn: float      # fraction of the history set redrawn per step
    steps: int
    grow: bool        # context grows by one token per step
    seed: int
    grow_per: int = 1  # tokens per unit: with grow, the context at step t is ctx + ceil(t / grow_per) units

    def ctx_at(self, t: int) -> int:
        return self.ctx + (-(-t // self.grow_per) if self.grow else 0)

    @property
    def ctx_max(self) -> int:
        return self.ctx_at(self.steps)

    @property
    def hist(self) -> int:
        return self.k - self.window


def _zipf_cdf(N: int, s: float) -> np.ndarray:
    w = np.arange(1, N + 1, dtype=np.float64) ** (-s)
    c = np.cumsum(w)
    return c / c[-1]


class _Req:
    def __init__(self, spec: TraceSpec, r: int, cdf: np.ndarray):
        self.spec = spec
        self.rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([spec.seed, r])))
        self.perm = self.rng.permutation(spec.ctx_max).astype(np.int64)
        self.cdf = cdf
        self.in_set = np.zeros(spec.ctx_max, dtype=bool)
        self.hist = np.empty(0, dtype=np.int64)

    def _draw(self, need: int, limit: int) -> np.ndarray:
        got = []
        while need > 0:
            u = self.rng.random(max(2 * need, 64))
            ranks = np.minimum(np.searchsorted(self.cdf, u, side="right"), self.cdf.size - 1)
            pos = self.perm[ranks]
            pos = pos[pos < limit]
            _, first = np.unique(pos, return_index=True)
            pos = pos[np.sort(first)]
            pos = pos[~self.in_set[pos]][:need]
            self.in_set[pos] = True
            got.append(pos)
            need -= pos.size
        return np.concatenate(got) if got else np.empty(0, dtype=np.int64)

    def step(self, t: int) -> np.ndarray:
        sp = self.spec
        L_t = sp.ctx_at(t)
        limit = L_t - sp.window
        if t == 0:
            self.hist = self._draw(sp.hist, limit)
        else:
            c = int(np.floor(sp.churn * sp.hist + 0.5))
            if c:
                drop = self.rng.choice(self.hist.size, size=c, replace=False)
                self.in_set[self.hist[drop]] = False
                self.hist = np.delete(self.hist, drop)
                self.hist = np.concatenate([self.hist, self._draw(c, limit)])
        sel = np.concatenate([self.hist, np.arange(limit, L_t, dtype=np.int64)])
        return sel[self.rng.permutation(sel.size)]


def generate(spec: TraceSpec, steps: int | None = None, requests: int | None = None) -> np.ndarray:
    """int32 trace [steps][n][k]; optionally only the first ``steps`` / ``requests``."""
    T = spec.steps if steps is None else min(steps, spec.steps)
    n = spec.n if requests is None else min(requests, spec.n)
    if spec.window > spec.k or spec.window < 0:
        raise ValueError("window must lie in [0, k]")
    if spec.ctx - spec.window < spec.hist:
        raise ValueError("context too short for the history set")
    cdf = _zipf_cdf(spec.ctx_max, spec.zipf_s)
    out = np.empty((T, n, spec.k), dtype=np.int32)
    for r in range(n):
        req = _Req(spec, r, cdf)
        for t in range(T):
            out[t, r] = req.step(t)
    return out
