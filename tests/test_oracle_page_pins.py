"""Pins of the oracle's page-granular mode (paper abstract: the method is evaluated with the
NSA and Quest families, whose selections are blocks of consecutive tokens).

A page c holds tokens cP .. cP + P - 1; the page table maps pages to slots and a miss fetches
the page's P rows.  The pins tie the page mode to the token mode, which
tests/test_oracle_pins.py pins on its own:
  * whole pages: selecting every token of a set of pages in token mode, with B * P slots,
    leaves exactly the page-mode state expanded -- slot group j holds page RM[j] in position
    order, with the page's stamp -- because candidates sorted by (stamp, slot) come in whole
    aligned groups and misses in ascending token order come in whole pages (LRU and FIFO);
  * a resident page's slot holds the P history rows of that page;
  * attention over pages equals attention over the same positions gathered straight from
    the history (only placement changes), cut at the context length, and it is the
    log-sum-exp merge of the attentions over each page alone;
  * append writes the new row through to the history and to its resident page's slot,
    leaves every table alone, and a page that was not resident arrives with the row.
Each fails for a plausible slip: the page's rows taken from the wrong offset, a slot
indexed in tokens instead of pages, a dropped or extra token at the length cut (< vs <=),
a page counted once instead of P times.
"""
import numpy as np
import pytest

import oracle
from synth import kv as skv


def _page_trace(rng, n, cap_pages, k, steps, pad=0.1):
    S = np.stack([np.stack([rng.choice(cap_pages, k, replace=False) for _ in range(n)]) for _ in range(steps)])
    S = S.astype(np.int32)
    S[rng.random(S.shape) < pad] = -1
    return S


def _expand(S, P):
    """Token selection naming every token of each selected page (padding stays padding)."""
    n, k = S.shape
    out = np.full((n, k * P), -1, dtype=np.int32)
    for r in range(n):
        for i in range(k):
            if S[r, i] >= 0:
                out[r, i * P:(i + 1) * P] = S[r, i] * P + np.arange(P)
    return out


@pytest.mark.parametrize("policy", [oracle.LRU, oracle.FIFO])
@pytest.mark.parametrize("P,B,cap_pages,k", [(2, 6, 30, 4), (4, 10, 40, 7), (8, 5, 25, 5), (16, 3, 12, 2)])
def test_whole_pages_equal_token_mode(policy, P, B, cap_pages, k):
    rng = np.random.default_rng(P * 100 + B + policy)
    n, L = 2, 1
    host = rng.integers(0, 256, size=(n, L, cap_pages * P, 1152), dtype=np.uint8)
    pg = oracle.OracleCache(n, L, B, cap_pages, host=host, policy=policy, page_tokens=P)
    tk = oracle.OracleCache(n, L, B * P, cap_pages * P, host=host.copy(), policy=policy)
    for S in _page_trace(rng, n, cap_pages, k, 40):
        s_pg, m_pg = pg.resolve(0, S)
        s_tk, m_tk = tk.resolve(0, _expand(S, P))
        assert (m_tk == P * m_pg).all()
        for r in range(n):
            for i in range(k):
                want = -1 if s_pg[r, i] < 0 else s_pg[r, i] * P + np.arange(P)
                assert (s_tk[r, i * P:(i + 1) * P] == want).all()
            PT = pg.PT[r, 0]
            exp_pt = np.where(np.repeat(PT, P) >= 0, np.repeat(PT, P) * P + np.tile(np.arange(P), cap_pages), -1)
            assert (tk.PT[r, 0] == exp_pt).all()
            RM = pg.RM[r, 0]
            exp_rm = np.where(np.repeat(RM, P) >= 0, np.repeat(RM, P) * P + np.tile(np.arange(P), B), -1)
            assert (tk.RM[r, 0] == exp_rm).all()
            assert (tk.ST[r, 0] == np.repeat(pg.ST[r, 0], P)).all()
        assert (tk.dev.reshape(pg.dev.shape) == pg.dev).all()


@pytest.mark.parametrize("policy", [oracle.LRU, oracle.FIFO, oracle.RANDOM])
def test_resident_page_holds_its_history_rows(policy):
    rng = np.random.default_rng(7 + policy)
    n, L, B, P, cap_pages, k = 3, 2, 9, 4, 40, 6
    host = rng.integers(0, 256, size=(n, L, cap_pages * P, 656), dtype=np.uint8)
    oc = oracle.OracleCache(n, L, B, cap_pages, layout=1, host=host, policy=policy, seed=3, page_tokens=P)
    for t in range(30):
        for layer in range(L):
            S = _page_trace(rng, n, cap_pages, k, 1)[0]
            before = oc.PT[:, layer].copy()
            slots, miss = oc.resolve(layer, S)
            for r in range(n):
                valid = S[r][S[r] >= 0]
                assert int(miss[r]) == int((before[r, valid] < 0).sum())
                assert len(set(slots[r][S[r] >= 0])) == len(valid)
                for j in np.nonzero(oc.RM[r, layer] >= 0)[0]:
                    c = int(oc.RM[r, layer, j])
                    assert oc.PT[r, layer, c] == j
                    assert (oc.dev[r, layer, j] == host[r, layer, c * P:(c + 1) * P].reshape(-1)).all()


def test_page_tokens_one_is_token_mode():
    rng = np.random.default_rng(2)
    host = rng.integers(0, 256, size=(2, 1, 50, 1152), dtype=np.uint8)
    a = oracle.OracleCache(2, 1, 8, 50, host=host)
    b = oracle.OracleCache(2, 1, 8, 50, host=host.copy(), page_tokens=1)
    for S in _page_trace(rng, 2, 50, 5, 20):
        sa, ma = a.resolve(0, S)
        sb, mb = b.resolve(0, S)
        assert (sa == sb).all() and (ma == mb).all()
    assert (a.PT == b.PT).all() and (a.dev == b.dev).all()


def _history(n, L, tokens, layout, seed):
    return np.stack([np.stack([skv.pool(seed, r, l, tokens, layout) for l in range(L)]) for r in range(n)])


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("P", [4, 16])
def test_attend_pages_equals_gather_from_history(layout, P):
    rng = np.random.default_rng(40 + P + layout)
    n, B, cap_pages, k, H = 3, 12, 20, 5, 4
    host = _history(n, 1, cap_pages * P, layout, 11)
    oc = oracle.OracleCache(n, 1, B, cap_pages, layout=layout, host=host, page_tokens=P)
    scale = 1.0 / np.sqrt(576.0)
    for t in range(6):
        S = _page_trace(rng, n, cap_pages, k, 1, pad=0.15)[0]
        slots, _ = oc.resolve(0, S)
        lens = rng.integers(1, cap_pages * P + 1, size=n)
        lens[0] = cap_pages * P
        q = skv.queries(5, t, n, 0, H)
        out, lse = oc.attend_pages(0, q, slots, S, lens, scale)
        # the same positions read from the full history, in the same order
        pos = np.full((n, k * P), -1, dtype=np.int32)
        for r in range(n):
            for i in range(k):
                for o in range(P):
                    if S[r, i] >= 0 and S[r, i] * P + o < lens[r]:
                        pos[r, i * P + o] = S[r, i] * P + o
        want_o, want_l = oracle.attend_rows(q, pos, host[:, 0], layout, scale)
        assert np.array_equal(out, want_o) and np.array_equal(lse, want_l)
        # whole pages when no length is given
        out_all, _ = oc.attend(0, q, slots, scale)
        full = np.where(np.repeat(S, P, axis=1) >= 0, np.repeat(S, P, axis=1) * P + np.tile(np.arange(P), k), -1)
        want_all, _ = oracle.attend_rows(q, full.astype(np.int32), host[:, 0], layout, scale)
        assert np.array_equal(out_all, want_all)


def test_length_cut_excludes_exactly_the_positions_past_the_end():
    # history rows at and past the length are NaN: any of them taken makes the output NaN
    P, n, B, cap_pages, k, H = 8, 2, 6, 6, 3, 2
    host = _history(n, 1, cap_pages * P, 0, 3)
    oc = oracle.OracleCache(n, 1, B, cap_pages, host=host, page_tokens=P)
    S = np.array([[5, 2, 0], [1, 3, 4]], dtype=np.int32)
    slots, _ = oc.resolve(0, S)
    lens = np.array([5 * P + 3, 4 * P + 1])
    poisoned = oc.dev.copy()
    for r in range(n):
        for j in range(B):
            c = int(oc.RM[r, 0, j])
            for o in range(P):
                if c >= 0 and c * P + o >= lens[r]:
                    poisoned[r, 0, j, o * 1152:(o + 1) * 1152] = np.frombuffer(
                        np.full(576, 0x7FC0, dtype=np.uint16).tobytes(), dtype=np.uint8)
    oc.dev = poisoned
    q = skv.queries(1, 0, n, 0, H)
    out, lse = oc.attend_pages(0, q, slots, S, lens, 0.05)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    lens2 = lens + 1                                        # one more position: a NaN row joins
    out2, _ = oc.attend_pages(0, q, slots, S, lens2, 0.05)
    assert np.isnan(out2).all()


def test_page_attention_is_lse_merge_of_single_pages():
    rng = np.random.default_rng(9)
    P, n, B, cap_pages, k, H = 4, 2, 8, 16, 6, 3
    host = _history(n, 1, cap_pages * P, 1, 21)
    oc = oracle.OracleCache(n, 1, B, cap_pages, layout=1, host=host, page_tokens=P)
    S = _page_trace(rng, n, cap_pages, k, 1, pad=0.0)[0]
    slots, _ = oc.resolve(0, S)
    q = skv.queries(2, 0, n, 0, H)
    out, lse = oc.attend(0, q, slots, 0.04)
    parts = [oc.attend(0, q, slots[:, i:i + 1], 0.04) for i in range(k)]
    L = np.stack([p[1] for p in parts])                      # [k][n][H]
    M = np.logaddexp.reduce(L, axis=0)
    assert np.allclose(M, lse, rtol=0, atol=1e-12)
    merged = sum(np.exp(parts[i][1] - M)[..., None] * parts[i][0] for i in range(k))
    assert np.allclose(merged, out, rtol=0, atol=1e-12)


def test_page_append_writes_through_and_keeps_tables():
    # a resident page takes the new row at its offset; a page that is not resident is left to
    # the next miss, which fetches it whole with the new row; tables never change
    rng = np.random.default_rng(12)
    P, n, B, cap_pages, k = 4, 2, 5, 12, 3
    host = rng.integers(0, 256, size=(n, 1, cap_pages * P, 1152), dtype=np.uint8)
    oc = oracle.OracleCache(n, 1, B, cap_pages, host=host.copy(), page_tokens=P)
    oc.resolve(0, np.array([[2, 7, 9], [0, 1, -1]], dtype=np.int32))
    tables = (oc.PT.copy(), oc.RM.copy(), oc.ST.copy(), oc.t.copy())
    rows = rng.integers(0, 256, size=(n, 1152), dtype=np.uint8)
    slots = oc.append(0, np.array([7 * P + 3, 5 * P + 1]), rows)         # page 7 resident, page 5 not
    assert slots[0] == oc.PT[0, 0, 7] and slots[1] == -1
    for a, b in zip(tables, (oc.PT, oc.RM, oc.ST, oc.t)):
        assert (a == b).all()
    j = int(slots[0])
    assert (oc.dev[0, 0, j].reshape(P, 1152)[3] == rows[0]).all()
    assert (oc.host[0, 0, 7 * P + 3] == rows[0]).all() and (oc.host[1, 0, 5 * P + 1] == rows[1]).all()
    for r in range(n):                                                    # resident pages = history pages
        for jj in np.nonzero(oc.RM[r, 0] >= 0)[0]:
            c = int(oc.RM[r, 0, jj])
            assert (oc.dev[r, 0, jj] == oc.host[r, 0, c * P:(c + 1) * P].reshape(-1)).all()
    oc.resolve(0, np.array([[2, 7, 9], [5, 0, -1]], dtype=np.int32))     # page 5 now fetched with its new row
    j5 = int(oc.PT[1, 0, 5])
    assert (oc.dev[1, 0, j5].reshape(P, 1152)[1] == rows[1]).all()
    with pytest.raises(oracle.OracleError):
        oc.append(0, np.array([cap_pages * P, -1]), rows)
    assert oc.append(0, np.array([-1, -1]), rows).tolist() == [-1, -1]
