"""Pins of the CPU oracle against what the pages and the mathematics fix.

The resolver's rule (HiSparse paper abstract: hit detection, LRU replacement,
host-to-device fetch; "HiSparse" note, sections 2-3: a miss is swapped in and
the eviction candidate is picked by LRU, then the page table is updated) with
the tie rules stated in oracle/hs_oracle.c.  Each pin below would fail for a
plausible slip in the oracle: misses taken in selection order instead of
ascending token order, a wrong tie-break, hits not refreshing recency, a hit
slot chosen as victim, the evicted token left in the page table, a dropped
attention term, a wrong E4M3 exponent bias.
"""
import itertools
import math
from collections import OrderedDict

import numpy as np
import pytest
import torch

import oracle
from oracle.naive import NaiveState
from synth import kv as skv


def _single(B, cap, layout=0, host=None):
    return oracle.OracleCache(1, 1, B, cap, layout=layout, host=host)


def _res(oc, S):
    slots, miss = oc.resolve(0, np.asarray([S], dtype=np.int32))
    return list(slots[0]), int(miss[0])


# ---------------------------------------------------------------- hand-worked rule examples

def test_misses_ascending_and_lowest_slot_first():
    # Empty buffer: every slot has stamp -1, so slots go out lowest index first,
    # and misses are served in ascending token order (5 arrives first, gets slot 1).
    oc = _single(B=4, cap=16)
    slots, m = _res(oc, [5, 3])
    assert (slots, m) == ([1, 0], 2)
    assert oc.PT[0, 0, 3] == 0 and oc.PT[0, 0, 5] == 1
    assert list(oc.RM[0, 0]) == [3, 5, -1, -1]
    assert list(oc.ST[0, 0]) == [0, 0, -1, -1]


def test_worked_sequence():
    oc = _single(B=4, cap=16)
    assert _res(oc, [5, 3]) == ([1, 0], 2)
    # t=1: 5 hits slot 1; 7 misses; non-hit slots by (stamp, slot): (-1,2) (-1,3) (0,0)
    assert _res(oc, [7, 5]) == ([2, 1], 1)
    assert list(oc.ST[0, 0]) == [0, 1, 1, -1]
    # t=2: 3 hits slot 0; misses 8 < 9; candidates (-1,3) (1,1) (1,2): 8->3, 9->1 evicting 5
    assert _res(oc, [9, 8, 3]) == ([1, 3, 0], 2)
    assert oc.PT[0, 0, 5] == -1
    assert list(oc.RM[0, 0]) == [3, 9, 7, 8]
    assert list(oc.ST[0, 0]) == [2, 2, 1, 2]
    # t=3: padding skipped; 5 misses and takes slot 2 (stamp 1 is the oldest), evicting 7
    assert _res(oc, [5, -1]) == ([2, -1], 1)
    assert oc.PT[0, 0, 7] == -1
    assert list(oc.RM[0, 0]) == [3, 9, 5, 8]
    assert list(oc.ST[0, 0]) == [2, 2, 3, 2]
    assert list(oc.t[0]) == [4]


def test_hit_refreshes_recency():
    oc = _single(B=2, cap=8)
    _res(oc, [1]); _res(oc, [2]); _res(oc, [1])
    # token 2 (stamp 1) is now least recent; token 1 was refreshed at step 2
    assert _res(oc, [3]) == ([1], 1)
    assert oc.PT[0, 0, 2] == -1 and oc.PT[0, 0, 1] == 0


def test_hit_slot_never_victim():
    oc = _single(B=3, cap=8)
    _res(oc, [1]); _res(oc, [2]); _res(oc, [3])
    # token 1's slot is the least recently used, but 1 is selected again: 4 must take slot 1
    assert _res(oc, [1, 4]) == ([0, 1], 1)
    assert oc.PT[0, 0, 2] == -1 and oc.PT[0, 0, 1] == 0


def test_invalid_selections_rejected_state_untouched():
    oc = _single(B=4, cap=8)
    _res(oc, [1, 2])
    before = (oc.PT.copy(), oc.RM.copy(), oc.ST.copy(), oc.t.copy())
    for bad in ([1, 1], [8, 0], [-2, 0], [3, 3, 3]):
        with pytest.raises(oracle.OracleError):
            oc.resolve(0, np.asarray([bad + [-1] * (3 - len(bad))], dtype=np.int32))
    for a, b in zip(before, (oc.PT, oc.RM, oc.ST, oc.t)):
        assert (a == b).all()


# ---------------------------------------------------------------- textbook LRU (k = 1)

class _TextbookLRU:
    def __init__(self, cap):
        self.cap, self.d = cap, OrderedDict()

    def access(self, key):
        if key in self.d:
            self.d.move_to_end(key)
            return True
        if len(self.d) >= self.cap:
            self.d.popitem(last=False)
        self.d[key] = True
        return False


@pytest.mark.parametrize("B", [1, 2, 3, 8, 17])
def test_k1_equals_textbook_lru(B):
    rng = np.random.default_rng(B)
    cap = 40
    oc = _single(B=B, cap=cap)
    ref = _TextbookLRU(B)
    seq = rng.zipf(1.3, size=3000) % cap
    for s in seq:
        _, m = _res(oc, [int(s)])
        assert (m == 0) == ref.access(int(s))
        resident = set(np.nonzero(oc.PT[0, 0] >= 0)[0].tolist())
        assert resident == set(ref.d.keys())


def test_k1_hit_counts_equal_functools_lru_cache():
    import functools
    B, cap = 7, 30
    rng = np.random.default_rng(5)
    seq = [int(x) for x in rng.zipf(1.2, size=2000) % cap]

    @functools.lru_cache(maxsize=B)
    def f(x):
        return x

    oc = _single(B=B, cap=cap)
    hits = 0
    for s in seq:
        f(s)
        hits += (_res(oc, [s])[1] == 0)
    assert hits == f.cache_info().hits


# ---------------------------------------------------------------- closed forms

def test_constant_selection():
    oc = _single(B=64, cap=1000)
    S = list(np.random.default_rng(1).choice(1000, 40, replace=False))
    ms = [_res(oc, S)[1] for _ in range(10)]
    assert ms == [40] + [0] * 9


def test_compulsory_misses_only_when_universe_fits():
    rng = np.random.default_rng(2)
    B, cap = 32, 500
    universe = rng.choice(cap, B, replace=False)
    oc = _single(B=B, cap=cap)
    seen = set()
    for _ in range(60):
        S = rng.choice(universe, 10, replace=False)
        _, m = _res(oc, list(S))
        assert m == len(set(S.tolist()) - seen)
        seen |= set(S.tolist())
    assert (oc.RM[0, 0] >= 0).sum() == len(seen)


@pytest.mark.parametrize("B,k", [(8, 8), (12, 5), (40, 16)])
def test_sliding_window(B, k):
    oc = _single(B=B, cap=400)
    prev_resident = set()
    for t in range(200):
        S = list(range(t, t + k))
        _, m = _res(oc, S[::-1])
        assert m == (k if t == 0 else 1)
        resident = set(np.nonzero(oc.PT[0, 0] >= 0)[0].tolist())
        if t + k > B:
            evicted = prev_resident - resident
            assert evicted == {t + k - 1 - B}
        assert resident == set(range(max(0, t + k - B), t + k))
        prev_resident = resident


def test_buffer_equal_to_k_holds_exactly_the_selection():
    rng = np.random.default_rng(3)
    k, cap = 12, 80
    oc = _single(B=k, cap=cap)
    for _ in range(100):
        S = rng.choice(cap, k, replace=False)
        _res(oc, list(S))
        assert set(np.nonzero(oc.PT[0, 0] >= 0)[0].tolist()) == set(S.tolist())


# ---------------------------------------------------------------- brute force over orders

@pytest.mark.parametrize("seed", range(6))
def test_all_presentation_orders_agree(seed):
    rng = np.random.default_rng(seed)
    B, cap, k = 6, 14, 5
    prefix = [list(rng.choice(cap, k, replace=False)) for _ in range(4)]
    S = list(rng.choice(cap, k, replace=False))
    if seed % 2:
        S[rng.integers(k)] = -1
    ref = None
    for perm in itertools.permutations(range(k)):
        host = np.arange(cap * 1152, dtype=np.uint64).astype(np.uint8).reshape(1, 1, cap, 1152)
        oc = oracle.OracleCache(1, 1, B, cap, layout=0, host=np.ascontiguousarray(host))
        for p in prefix:
            _res(oc, p)
        Sp = [S[i] for i in perm]
        slots, m = _res(oc, Sp)
        state = (oc.PT.tobytes(), oc.RM.tobytes(), oc.ST.tobytes(), oc.dev.tobytes(), m)
        by_token = {s: sl for s, sl in zip(Sp, slots) if s != -1}
        if ref is None:
            ref = (state, by_token)
        else:
            assert state == ref[0]
            assert by_token == ref[1]


# ---------------------------------------------------------------- second implementation

def _check_same(oc, nv):
    PT, RM, ST = nv.arrays()
    assert list(oc.PT[0, 0]) == PT
    assert list(oc.RM[0, 0]) == RM
    assert list(oc.ST[0, 0]) == ST


def test_naive_agrees_exhaustive_two_steps():
    cap, B = 6, 3
    subsets = [list(c) for r in range(0, 4) for c in itertools.combinations(range(cap), r)]
    for a in subsets:
        for b in subsets:
            oc, nv = _single(B, cap), NaiveState(B, cap)
            for S in (a, b, [5, 0, 2]):
                Sp = S + [-1] * (3 - len(S))
                got = _res(oc, Sp)
                want = nv.resolve(Sp)
                assert got == want
            _check_same(oc, nv)


@pytest.mark.parametrize("seed", range(8))
def test_naive_agrees_random(seed):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(4, 40))
    k = int(rng.integers(1, B + 1))
    cap = int(rng.integers(B + 1, 4 * B + 8))
    oc, nv = _single(B, cap), NaiveState(B, cap)
    for _ in range(80):
        S = list(rng.choice(cap, k, replace=False))
        for i in range(k):
            if rng.random() < 0.1:
                S[i] = -1
        slots, m = _res(oc, S)
        slots2, m2 = nv.resolve(S)
        assert (slots, m) == (slots2, m2)
    _check_same(oc, nv)


# ---------------------------------------------------------------- invariants on traces

def _check_invariants(oc, S, slots, m, prev_resident, last_use, t, host):
    PT, RM, ST = oc.PT[0, 0], oc.RM[0, 0], oc.ST[0, 0]
    valid = [s for s in S if s != -1]
    # every selected token resident, slot mapping consistent, output slots right
    for s, sl in zip(S, slots):
        if s == -1:
            assert sl == -1
        else:
            assert PT[s] == sl and RM[sl] == s and ST[sl] == t
    # PT and RM are inverse bijections
    res = np.nonzero(PT >= 0)[0]
    assert len(set(PT[res].tolist())) == res.size
    assert all(RM[PT[x]] == x for x in res)
    occ = np.nonzero(RM >= 0)[0]
    assert all(PT[RM[j]] == j for j in occ)
    # miss count = |S \ resident before|; hits + misses = |valid S|
    assert m == len(set(valid) - prev_resident)
    hits = len(set(valid) & prev_resident)
    assert hits + m == len(valid)
    # no selected token was evicted; stamps never exceed the step
    resident = set(res.tolist())
    assert set(valid) <= resident
    assert (ST <= t).all()
    # slot bytes equal the host row of their owner
    for j in occ:
        assert (oc.dev[0, 0, j] == host[0, 0, RM[j]]).all()
    # recency: resident tokens were used no earlier than any evicted one
    for s in valid:
        last_use[s] = t
    evicted_seen = [x for x in last_use if x not in resident]
    if evicted_seen and resident:
        assert min(int(ST[PT[x]]) for x in resident) >= max(last_use[x] for x in evicted_seen)
    return resident


@pytest.mark.parametrize("B,k,cap,steps", [(16, 8, 64, 120), (32, 32, 100, 60), (48, 20, 300, 150)])
def test_invariants_random_traces(B, k, cap, steps):
    rng = np.random.default_rng(B * 1000 + k)
    host = rng.integers(0, 256, size=(1, 1, cap, 1152), dtype=np.uint8)
    oc = oracle.OracleCache(1, 1, B, cap, layout=0, host=host)
    resident, last_use = set(), {}
    pop = rng.permutation(cap)
    w = 1.0 / np.arange(1, cap + 1) ** 1.1
    w /= w.sum()
    for t in range(steps):
        S = list(rng.choice(pop, k, replace=False, p=w))
        for i in range(k):
            if rng.random() < 0.05:
                S[i] = -1
        slots, m = _res(oc, S)
        resident = _check_invariants(oc, S, slots, m, resident, last_use, t, host)


@pytest.mark.parametrize("policy", [oracle.LRU, oracle.FIFO])
def test_relabelled_steps_give_same_placement(policy):
    # Any strictly increasing step numbering gives the same placement (for the stamp-ordered
    # policies; RANDOM keys its permutation by the step number itself).
    rng = np.random.default_rng(9)
    B, cap, k = 20, 90, 9
    seq = [np.asarray(rng.choice(cap, k, replace=False), dtype=np.int32) for _ in range(50)]
    L = oracle.lib()
    states = []
    for stride in (1, 7):
        PT = np.full(cap, -1, np.int32); RM = np.full(B, -1, np.int32); ST = np.full(B, -1, np.int64)
        slots = np.empty(k, np.int32); miss = np.empty(1, np.int64)
        for t, S in enumerate(seq):
            assert L.orc_resolve(B, cap, k, PT.ctypes.data, RM.ctypes.data, ST.ctypes.data, 100 + t * stride,
                                 S.ctypes.data, slots.ctypes.data, miss.ctypes.data, None, None, 1152,
                                 policy, 0, 0) == 0
        states.append((PT.copy(), RM.copy()))
    assert (states[0][0] == states[1][0]).all() and (states[0][1] == states[1][1]).all()


# ---------------------------------------------------------------- E4M3 decode

def test_e4m3_decode_matches_torch_table():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_decode(c) for c in range(256)])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert (got[~nan] == ref[~nan]).all()
    assert np.nanmax(got) == 448.0 and np.isfinite(got[~nan]).all()


# ---------------------------------------------------------------- attention

def _decode_rows_torch(rows, layout):
    """Library decode of entries to (K[.,576], V[.,512]) in float64."""
    t = torch.from_numpy(np.ascontiguousarray(rows))
    if layout == 0:
        K = t.view(torch.bfloat16).reshape(-1, 576).to(torch.float64)
    else:
        lat = t[:, :512].contiguous().view(torch.float8_e4m3fn).to(torch.float64)
        sc = t[:, 512:528].contiguous().view(torch.float32).to(torch.float64)
        lat = lat * sc.repeat_interleave(128, dim=1)
        rope = t[:, 528:656].contiguous().view(torch.bfloat16).to(torch.float64)
        K = torch.cat([lat, rope], dim=1)
    return K, K[:, :512]


def _q_f64(q):
    return torch.from_numpy(q.astype(np.uint16).view(np.int16)).view(torch.bfloat16).to(torch.float64)


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("k", [1, 7, 64])
def test_attention_matches_torch_sdpa_fp64(layout, k):
    rng = np.random.default_rng(k + 10 * layout)
    R, H = 96, 16
    rows = skv.rows_at(77, 0, 0, np.arange(R), layout)[None]
    q = skv.queries(77, 3, 1, 0, H)
    idx = rng.choice(R, k, replace=False).astype(np.int32)[None]
    scale = 1.0 / math.sqrt(576)
    out, lse = oracle.attend_rows(q, idx, rows, layout, scale)
    K, V = _decode_rows_torch(rows[0][idx[0]], layout)
    Q = _q_f64(q[0])
    ref = torch.nn.functional.scaled_dot_product_attention(Q[None], K[None], V[None], scale=scale)
    ref = ref[0].numpy()
    assert np.abs(out[0] - ref).max() < 1e-12
    s = (Q @ K.T) * scale
    ref_lse = torch.logsumexp(s, dim=1).numpy()
    assert np.abs(lse[0] - ref_lse).max() < 1e-12


def test_attention_single_entry_is_its_value_row():
    rows = skv.rows_at(5, 0, 0, np.arange(10), 1)[None]
    q = skv.queries(5, 0, 1, 0, 4)
    out, lse = oracle.attend_rows(q, np.array([[-1, 6, -1]], np.int32), rows, 1, 0.05)
    _, V = _decode_rows_torch(rows[0][[6]], 1)
    assert (out[0] == V.numpy()[0][None, :]).all()


def test_attention_zero_query_averages_values():
    rows = skv.rows_at(6, 0, 0, np.arange(30), 0)[None]
    q = np.zeros((1, 3, 576), np.uint16)
    idx = np.array([[3, 11, -1, 29, 0]], np.int32)
    out, lse = oracle.attend_rows(q, idx, rows, 0, 0.1)
    _, V = _decode_rows_torch(rows[0][[3, 11, 29, 0]], 0)
    assert np.abs(out[0] - V.numpy().mean(axis=0)[None]).max() < 1e-15
    assert np.abs(lse[0] - math.log(4)).max() < 1e-15


def test_attention_no_valid_entry():
    rows = skv.rows_at(6, 0, 0, np.arange(4), 0)[None]
    q = skv.queries(6, 0, 1, 0, 2)
    out, lse = oracle.attend_rows(q, np.full((1, 5), -1, np.int32), rows, 0, 0.1)
    assert (out == 0).all() and np.isneginf(lse).all()


@pytest.mark.parametrize("layout", [0, 1])
def test_exactness_resolved_slots_equal_direct_gather(layout):
    """Only placement changes: attention over resolved slots == attention over the host rows."""
    rng = np.random.default_rng(layout)
    n, B, cap, k, H = 3, 24, 120, 16, 16
    host = np.stack([skv.pool(11, r, 0, cap, layout) for r in range(n)])[:, None]
    oc = oracle.OracleCache(n, 1, B, cap, layout=layout, host=np.ascontiguousarray(host))
    for t in range(25):
        S = np.stack([rng.choice(cap, k, replace=False) for _ in range(n)]).astype(np.int32)
        S[rng.random(S.shape) < 0.1] = -1
        slots, _ = oc.resolve(0, S)
        q = skv.queries(11, t, n, 0, H)
        o1, l1 = oc.attend(0, q, slots, 0.0416)
        o2, l2 = oracle.attend_rows(q, S, host[:, 0], layout, 0.0416)
        assert o1.tobytes() == o2.tobytes() and l1.tobytes() == l2.tobytes()
