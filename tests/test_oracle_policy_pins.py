"""Pins of the oracle's eviction-policy variants (the HiSparse note, section 3: the miss-count
experiment varies the buffer size and the eviction policy, and LRU is steadier than a policy
that does not exploit locality).

FIFO: candidates by (fill stamp, slot) -- a hit does not refresh a slot.  RANDOM: the non-hit
slots in slot order, the i-th miss taking candidate perm(i) of a keyed pseudo-random
permutation (Feistel network with cycle walking over SplitMix64 outputs).  Each pin fails for a
plausible slip: FIFO refreshing on hits, a wrong tie-break, a permutation that is not a
bijection or not keyed by the step, a RANDOM victim that holds a hit.
"""
from collections import OrderedDict, deque

import numpy as np
import pytest

import oracle
from oracle import naive
from oracle.naive import NaiveState

BELADY = [1, 2, 3, 4, 1, 2, 5, 1, 2, 3, 4, 5]


def _faults(policy, B, refs, cap=16):
    oc = oracle.OracleCache(1, 1, B, cap, policy=policy)
    return sum(int(oc.resolve(0, np.array([[p]], dtype=np.int32))[1][0]) for p in refs)


def test_fifo_belady_anomaly():
    # the textbook reference string: FIFO takes 9 faults with 3 frames and 10 with 4
    assert _faults(oracle.FIFO, 3, BELADY) == 9
    assert _faults(oracle.FIFO, 4, BELADY) == 10


def test_lru_on_belady_string():
    # LRU on the same string: 10 faults with 3 frames, 8 with 4 (no anomaly for a stack policy)
    assert _faults(oracle.LRU, 3, BELADY) == 10
    assert _faults(oracle.LRU, 4, BELADY) == 8


@pytest.mark.parametrize("B", [1, 2, 5, 9])
def test_fifo_k1_equals_textbook_queue(B):
    rng = np.random.default_rng(B)
    refs = rng.integers(0, 3 * B + 2, size=400).tolist()
    q, resident, faults = deque(), set(), 0
    for p in refs:
        if p not in resident:
            faults += 1
            if len(q) == B:
                resident.discard(q.popleft())
            q.append(p)
            resident.add(p)
    assert _faults(oracle.FIFO, B, refs, cap=3 * B + 2) == faults


@pytest.mark.parametrize("B", [2, 6])
def test_lru_k1_equals_ordered_dict(B):
    rng = np.random.default_rng(10 + B)
    refs = rng.integers(0, 3 * B, size=300).tolist()
    od, faults = OrderedDict(), 0
    for p in refs:
        if p in od:
            od.move_to_end(p)
        else:
            faults += 1
            if len(od) == B:
                od.popitem(last=False)
            od[p] = True
    assert _faults(oracle.LRU, B, refs, cap=3 * B) == faults


def test_fifo_hit_does_not_refresh():
    # B = 2: fill 1 then 2; hit 1; miss 3 evicts 1 under FIFO (oldest fill) but 2 under LRU
    for policy, evicted in ((oracle.FIFO, 1), (oracle.LRU, 2)):
        oc = oracle.OracleCache(1, 1, 2, 8, policy=policy)
        for p in (1, 2, 1, 3):
            oc.resolve(0, np.array([[p]], dtype=np.int32))
        assert oc.PT[0, 0, evicted] == -1 and oc.PT[0, 0, 3] >= 0
    oc = oracle.OracleCache(1, 1, 2, 8, policy=oracle.FIFO)
    for p in (1, 2, 1):
        oc.resolve(0, np.array([[p]], dtype=np.int32))
    assert list(oc.ST[0, 0]) == [0, 1]          # slot of 1 keeps its fill step 0


@pytest.mark.parametrize("N", list(range(1, 70)) + [255, 256, 257, 1000, 4096, 4097, 6144])
def test_random_perm_is_a_bijection(N):
    seed, rl, t = 1234567, 3, 17
    img = [oracle.random_perm(seed, rl, t, N, x) for x in range(N)]
    assert sorted(img) == list(range(N))


def test_random_perm_matches_second_statement_and_is_keyed():
    rng = np.random.default_rng(4)
    for _ in range(300):
        seed = int(rng.integers(0, 2**63))
        rl, t = int(rng.integers(0, 5000)), int(rng.integers(0, 100000))
        N = int(rng.integers(1, 20000))
        x = int(rng.integers(0, N))
        assert oracle.random_perm(seed, rl, t, N, x) == naive.random_perm(seed, rl, t, N, x)
    base = [oracle.random_perm(5, 0, 0, 1000, x) for x in range(20)]
    for other in ((6, 0, 0), (5, 1, 0), (5, 0, 1)):     # seed, request-layer and step all matter
        assert [oracle.random_perm(*other, 1000, x) for x in range(20)] != base


def test_random_first_victim_is_uniform():
    # over many steps the first miss's candidate rank is spread evenly over N candidates
    N, steps = 16, 16000
    counts = np.bincount([oracle.random_perm(99, 0, t, N, 0) for t in range(steps)], minlength=N)
    expected = steps / N
    chi2 = float(((counts - expected) ** 2 / expected).sum())
    assert chi2 < 45.0, counts          # 15 degrees of freedom: p < 1e-4 beyond ~45


@pytest.mark.parametrize("policy,name", [(oracle.LRU, "lru"), (oracle.FIFO, "fifo"), (oracle.RANDOM, "random")])
@pytest.mark.parametrize("seed", range(4))
def test_policies_agree_with_second_statement(policy, name, seed):
    rng = np.random.default_rng(50 + seed)
    B, cap, k = 14, 70, 6
    oc = oracle.OracleCache(1, 1, B, cap, policy=policy, seed=777)
    nv = NaiveState(B, cap, policy=name, seed=777, rl=0)
    for _ in range(60):
        S = rng.choice(cap, k, replace=False).astype(np.int32)
        S[rng.random(k) < 0.2] = -1
        slots, miss = oc.resolve(0, S[None])
        s2, m2 = nv.resolve(list(S))
        assert list(slots[0]) == s2 and int(miss[0]) == m2
        PT, RM, ST = nv.arrays()
        assert list(oc.PT[0, 0]) == PT and list(oc.RM[0, 0]) == RM and list(oc.ST[0, 0]) == ST


@pytest.mark.parametrize("policy", [oracle.FIFO, oracle.RANDOM])
def test_policy_invariants_random_traces(policy):
    rng = np.random.default_rng(policy)
    n, B, cap, k = 3, 24, 120, 10
    host = rng.integers(0, 256, size=(n, 1, cap, 1152), dtype=np.uint8)
    oc = oracle.OracleCache(n, 1, B, cap, host=host, policy=policy, seed=5)
    for t in range(80):
        S = np.stack([rng.choice(cap, k, replace=False) for _ in range(n)]).astype(np.int32)
        hits_before = [set(np.nonzero(oc.PT[r, 0] >= 0)[0]) & set(S[r]) for r in range(n)]
        slots, miss = oc.resolve(0, S)
        for r in range(n):
            assert (slots[r] >= 0).all() and len(set(slots[r])) == k          # all resident, distinct
            assert int(miss[r]) == k - len(hits_before[r])
            occ = np.nonzero(oc.RM[r, 0] >= 0)[0]
            assert (oc.PT[r, 0, oc.RM[r, 0, occ]] == occ).all()                # bijection
            assert (oc.dev[r, 0, occ] == host[r, 0, oc.RM[r, 0, occ]]).all()    # slot bytes = rows


def test_random_rejects_append_and_bad_policy():
    oc = oracle.OracleCache(1, 1, 4, 8, policy=oracle.RANDOM)
    with pytest.raises(oracle.OracleError):
        oc.append(0, np.array([1], dtype=np.int32), np.zeros((1, 1152), dtype=np.uint8))
    bad = oracle.OracleCache(1, 1, 4, 8, policy=7)
    with pytest.raises(oracle.OracleError):
        bad.resolve(0, np.array([[1]], dtype=np.int32))


def test_fifo_append_of_resident_token_keeps_fill_step():
    oc = oracle.OracleCache(1, 1, 3, 8, policy=oracle.FIFO)
    oc.resolve(0, np.array([[4]], dtype=np.int32))
    oc.resolve(0, np.array([[5]], dtype=np.int32))
    j = int(oc.append(0, np.array([4], dtype=np.int32), np.zeros((1, 1152), dtype=np.uint8))[0])
    assert oc.ST[0, 0, j] == 0                     # 4 was filled at step 0; rewriting it is no refill
    nv = NaiveState(3, 8, policy="fifo")
    nv.resolve([4])
    nv.resolve([5])
    assert nv.append(4) == j and nv.stamp[j] == 0
