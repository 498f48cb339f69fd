"""Pins of the top-k oracle (oracle/topk.py): brute force over every k-subset, closed forms,
and the defining order property; each fails for a plausible slip (ties to the larger
position, ascending instead of descending scores, output not in position order, len
ignored, -inf mishandled)."""
import itertools

import numpy as np
import pytest

from oracle.topk import topk


def _brute(s, k):
    # the subset of size min(k, n) maximising the sorted score vector, then smallest positions
    n = len(s)
    best = None
    for sub in itertools.combinations(range(n), min(k, n)):
        key = (sorted((s[i] for i in sub), reverse=True), [-i for i in sub])
        if best is None or key > best[0]:
            best = (key, sub)
    return list(best[1])


@pytest.mark.parametrize("seed", range(30))
def test_brute_force_small(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 9))
    k = int(rng.integers(1, 6))
    s = rng.integers(-3, 4, size=n).astype(np.float32)          # many ties on purpose
    if rng.random() < 0.3:
        s[rng.integers(0, n)] = -np.inf
    got = topk(s[None], np.array([n]), k)[0]
    want = _brute(list(s), k)
    assert list(got[: len(want)]) == want and (got[len(want):] == -1).all()


def test_closed_forms():
    k = 5
    inc = np.arange(20, dtype=np.float32)[None]
    assert list(topk(inc, np.array([20]), k)[0]) == [15, 16, 17, 18, 19]     # increasing: the last k
    const = np.zeros((1, 20), dtype=np.float32)
    assert list(topk(const, np.array([20]), k)[0]) == [0, 1, 2, 3, 4]        # all tied: the first k
    assert list(topk(inc, np.array([3]), k)[0]) == [0, 1, 2, -1, -1]         # len < k: all, then -1
    assert list(topk(inc, np.array([0]), k)[0]) == [-1] * 5
    neg = -inc                                                               # decreasing: the first k
    assert list(topk(neg, np.array([20]), k)[0]) == [0, 1, 2, 3, 4]
    ninf = np.full((1, 8), -np.inf, dtype=np.float32)
    ninf[0, 6] = 1.0
    assert list(topk(ninf, np.array([8]), 3)[0]) == [0, 1, 6]


@pytest.mark.parametrize("seed", range(5))
def test_selected_dominate_unselected(seed):
    rng = np.random.default_rng(100 + seed)
    n, L, k = 3, 5000, 300
    s = rng.standard_normal((n, L)).astype(np.float32)
    s[:, rng.integers(0, L, 400)] = 0.5                        # a block of ties near the cut
    lens = np.array([L, L - 17, 250])
    out = topk(s, lens, k)
    for r in range(n):
        sel = out[r][out[r] >= 0]
        assert (np.diff(sel) > 0).all()                       # ascending positions
        assert sel.size == min(k, lens[r])
        rest = np.setdiff1d(np.arange(lens[r]), sel)
        if rest.size:
            lo = s[r, sel].min()
            assert s[r, rest].max() <= lo                     # nothing unselected scores higher
            tied_out = rest[s[r, rest] == lo]
            tied_in = sel[s[r, sel] == lo]
            if tied_out.size:
                assert tied_in.max() < tied_out.min()         # ties go to smaller positions
