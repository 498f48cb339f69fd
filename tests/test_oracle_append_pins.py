"""Pins of the oracle's write-through append (the note's introduction: inactive KV is
offloaded to host memory actively; paper abstract: every request's full KV history lives in
host memory).  Reading: an appended token's row is written to its history position, and the
token becomes resident before the next resolve -- in its own slot if it has one, otherwise
in the first slot by (stamp, slot) over all slots, empty slots first -- stamped with the
next resolve's step.  Each pin fails for a plausible slip: the wrong victim order, an
evicted token left in the page table, a stamp that is not refreshed, a row written to the
wrong slot or history position, the step counter advanced by an append.
"""
import numpy as np
import pytest

import oracle
from oracle.naive import NaiveState

E = 1152


def _state(B, cap, n=1):
    host = np.zeros((n, 1, cap, E), dtype=np.uint8)
    return oracle.OracleCache(n, 1, B, cap, layout=0, host=host)


def _row(v):
    return np.full(E, v, dtype=np.uint8)


def _append(oc, p, v):
    return int(oc.append(0, np.array([p], dtype=np.int32), _row(v)[None])[0])


def _res(oc, S):
    slots, miss = oc.resolve(0, np.asarray([S], dtype=np.int32))
    return list(slots[0]), int(miss[0])


def test_append_hand_worked():
    oc = _state(B=3, cap=10)
    # empty buffer: every stamp is -1, so the lowest slot; stamped with the next step (0)
    assert _append(oc, 4, 11) == 0
    assert list(oc.ST[0, 0]) == [0, -1, -1] and oc.PT[0, 0, 4] == 0 and int(oc.t[0, 0]) == 0
    assert (oc.host[0, 0, 4] == 11).all() and (oc.dev[0, 0, 0] == 11).all()
    # step 0: 4 hits; 7 misses and takes the first empty slot
    assert _res(oc, [4, 7]) == ([0, 1], 1)
    assert list(oc.ST[0, 0]) == [0, 0, -1]
    # next step is 1: 5 takes the empty slot 2
    assert _append(oc, 5, 12) == 2
    # a resident token keeps its slot; row and stamp are refreshed
    assert _append(oc, 4, 13) == 0
    assert (oc.dev[0, 0, 0] == 13).all() and (oc.host[0, 0, 4] == 13).all()
    assert list(oc.ST[0, 0]) == [1, 0, 1]
    # stamps [1, 0, 1]: slot 1 is the least recently used; its token 7 leaves the page table
    assert _append(oc, 9, 14) == 1
    assert oc.PT[0, 0, 7] == -1 and list(oc.RM[0, 0]) == [4, 9, 5]
    assert list(oc.ST[0, 0]) == [1, 1, 1]
    # step 1: everything appended is a hit
    assert _res(oc, [9, 5, 4]) == ([1, 2, 0], 0)
    assert int(oc.t[0, 0]) == 2


@pytest.mark.parametrize("B,k", [(9, 8), (12, 8), (33, 32)])
def test_sliding_window_with_append_never_misses(B, k):
    # S_t = the last k positions up to t.  Appending t before step t makes t resident; when
    # B > k some resident token was not selected at t - 1 (stamp <= t - 2), so the victim is
    # never in the window: no misses at all.  Without the append, token t is new at every
    # step: exactly one miss per step.
    steps = 3 * B
    a, b = _state(B, 4 * B), _state(B, 4 * B)
    for t in range(steps):
        S = list(range(max(0, t - k + 1), t + 1))
        _append(a, t, t % 251)
        assert _res(a, S)[1] == 0, t
        assert _res(b, S)[1] == 1, t


def test_append_rejects_out_of_range_and_leaves_state():
    oc = _state(B=4, cap=8)
    _res(oc, [1, 2])
    before = (oc.PT.copy(), oc.RM.copy(), oc.ST.copy())
    for p in (8, -2, 1 << 20):
        with pytest.raises(oracle.OracleError):
            oc.append(0, np.array([p], dtype=np.int32), _row(1)[None])
    assert all((x == y).all() for x, y in zip(before, (oc.PT, oc.RM, oc.ST)))


def test_append_padding_entry_is_skipped():
    oc = _state(B=4, cap=8, n=2)
    out = oc.append(0, np.array([-1, 3], dtype=np.int32), np.stack([_row(1), _row(2)]))
    assert list(out) == [-1, 0]
    assert (oc.PT[0] == -1).all() and oc.PT[1, 0, 3] == 0


@pytest.mark.parametrize("seed", range(6))
def test_append_naive_agrees_random(seed):
    rng = np.random.default_rng(seed)
    B, cap, k = 12, 60, 7
    oc = _state(B, cap)
    nv = NaiveState(B, cap)
    nxt = 0
    for _ in range(80):
        if rng.random() < 0.5:
            # a new token, or sometimes an already-resident one
            p = int(rng.integers(0, cap)) if rng.random() < 0.3 else nxt % cap
            nxt += 1
            v = int(rng.integers(0, 256))
            j = _append(oc, p, v)
            assert nv.append(p, v) == j
        else:
            S = rng.choice(cap, k, replace=False).astype(np.int32)
            S[rng.random(k) < 0.2] = -1
            slots, m = _res(oc, list(S))
            s2, m2 = nv.resolve(list(S))
            assert slots == s2 and m == m2
        PT, RM, ST = nv.arrays()
        assert list(oc.PT[0, 0]) == PT and list(oc.RM[0, 0]) == RM and list(oc.ST[0, 0]) == ST
        assert int(oc.t[0, 0]) == nv.t


@pytest.mark.parametrize("seed", range(3))
def test_append_rows_match_history(seed):
    # after random appends and resolves, every resident slot holds its token's history row
    rng = np.random.default_rng(100 + seed)
    B, cap, k = 16, 80, 6
    host = rng.integers(0, 256, size=(1, 1, cap, E), dtype=np.uint8)
    oc = oracle.OracleCache(1, 1, B, cap, layout=0, host=host)
    written = {}
    for t in range(60):
        p = int(rng.integers(0, cap))
        row = rng.integers(0, 256, size=E, dtype=np.uint8)
        oc.append(0, np.array([p], dtype=np.int32), row[None])
        written[p] = row
        oc.resolve(0, rng.choice(cap, k, replace=False).astype(np.int32)[None])
    for p, row in written.items():
        assert (oc.host[0, 0, p] == row).all()
    for j in range(B):
        tok = oc.RM[0, 0, j]
        if tok >= 0:
            assert (oc.dev[0, 0, j] == oc.host[0, 0, tok]).all()
            assert oc.PT[0, 0, tok] == j
