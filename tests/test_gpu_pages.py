"""Page-granular selections on the GPU against the oracle (paper abstract: the NSA and Quest
families select blocks of consecutive tokens).  Bit-exact: page table, owners, stamps, step
counters, output slots, miss counts and every byte of the resident pages, fused and split
resolves, LRU / FIFO / RANDOM.  Attention within the fp64 oracle's tolerance (max abs 2e-2 on
the bf16 output, 1e-3 on lse): over whole pages (hs_attend) and cut at the context length
(hs_attend_pages), with padding pages, ragged lengths and the full-size page workload.  The
page-granular append writes through to the history and to resident pages, bit-exact."""
import math

import numpy as np
import pytest
import torch

import hierarchical_kv_cache_hs_amd as hsa
import oracle
from synth import configs as C
from synth import kv as skv

from gpu_harness import Pair, say, trace_for

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

TOL_OUT = 2e-2
TOL_LSE = 1e-3
SCALE = 1.0 / math.sqrt(576)


def _compare(out_g, lse_g, out_o, lse_o, what):
    og = out_g.float().cpu().numpy().astype(np.float64)
    lg = lse_g.cpu().numpy().astype(np.float64)
    err = np.abs(og - out_o).max() if og.size else 0.0
    assert err <= TOL_OUT, f"{what}: max abs error {err}"
    fin = np.isfinite(lse_o)
    assert (np.isfinite(lg) == fin).all(), f"{what}: lse finiteness differs"
    if fin.any():
        lerr = np.abs(lg[fin] - lse_o[fin]).max()
        assert lerr <= TOL_LSE, f"{what}: lse error {lerr}"
    return err


def _q(qb):
    return torch.from_numpy(qb.view(np.int16)).cuda().view(torch.bfloat16)


def _page_trace(rng, n, cap, k, pad):
    S = np.stack([rng.choice(cap, k, replace=False) for _ in range(n)]).astype(np.int32)
    S[rng.random(S.shape) < pad] = -1
    return S


@pytest.mark.parametrize("layout", [hsa.LAYOUT_BF16, hsa.LAYOUT_FP8])
@pytest.mark.parametrize("P,k,B,ratio,n", [(4, 40, 64, 6, 3), (16, 32, 48, 8, 2), (64, 9, 16, 5, 2),
                                           (2, 300, 700, 3, 2)])
@pytest.mark.parametrize("split", [False, True])
def test_page_resolve_matches_oracle(layout, P, k, B, ratio, n, split):
    say(f"pages resolve: P {P}, k {k}, B {B}, ratio {ratio}, n {n}, layout {layout}, split {split}")
    rng = np.random.default_rng(P * 7 + k + layout)
    p = Pair(n, 1, k, B, ratio, layout, seed=17, split=split, page_tokens=P)
    try:
        for t in range(8):
            p.step(0, _page_trace(rng, n, ratio * B, k, 0.1), check_state=True)
        assert p.hs.device_error() == 0
    finally:
        p.close()


@pytest.mark.parametrize("policy", [hsa.EVICT_FIFO, hsa.EVICT_RANDOM])
def test_page_resolve_policies(policy):
    say(f"pages resolve, policy {policy}: P 8, k 24, B 40")
    rng = np.random.default_rng(60 + policy)
    p = Pair(3, 2, 24, 40, 6, hsa.LAYOUT_FP8, seed=4, policy=policy, policy_seed=99, page_tokens=8)
    try:
        for t in range(10):
            for layer in range(2):
                p.step(layer, _page_trace(rng, 3, 240, 24, 0.05), check_state=True)
    finally:
        p.close()


@pytest.mark.parametrize("layout", [hsa.LAYOUT_BF16, hsa.LAYOUT_FP8])
@pytest.mark.parametrize("P,k,B,heads,n", [(4, 50, 80, 16, 3), (16, 20, 40, 5, 2), (64, 6, 12, 16, 2),
                                           (16, 128, 256, 16, 2), (64, 256, 320, 16, 2)])
def test_page_attention_matches_oracle(layout, P, k, B, heads, n):
    say(f"pages attend: P {P}, k {k}, B {B}, heads {heads}, n {n}, layout {layout}")
    rng = np.random.default_rng(P + k + heads + layout)
    ratio = 4 if k * P <= 8192 else 2          # 16384 attended tokens: 8 or 16 splits
    cap = ratio * B
    p = Pair(n, 1, k, B, ratio, layout, seed=23, heads=heads, page_tokens=P)
    try:
        for t in range(3):
            S = _page_trace(rng, n, cap, k, 0.15)
            if n > 2:
                S[2] = -1                       # no valid page: out 0, lse -inf
            slots, _ = p.step(0, S, check_state=False)
            qb = skv.queries(23, t, n, 0, heads)
            d_slots = torch.from_numpy(slots).cuda()
            out, lse = p.hs.attend(0, _q(qb), d_slots, SCALE)
            out_o, lse_o = p.orc.attend(0, qb, slots, SCALE)
            torch.cuda.synchronize()
            _compare(out, lse, out_o, lse_o, f"step {t}: whole pages")
            # cut at ragged lengths, some inside a selected page, one before every page
            lens = rng.integers(1, cap * P + 1, size=n).astype(np.int32)
            valid = S[0][S[0] >= 0]
            if valid.size:
                lens[0] = int(valid.max()) * P + P // 2 + 1
            if n > 1:
                lens[1] = 0
            out2, lse2 = p.hs.attend_pages(0, _q(qb), d_slots, torch.from_numpy(S).cuda(),
                                           torch.from_numpy(lens).cuda(), SCALE)
            out_o2, lse_o2 = p.orc.attend_pages(0, qb, slots, S, lens, SCALE)
            torch.cuda.synchronize()
            _compare(out2, lse2, out_o2, lse_o2, f"step {t}: cut at the context length")
            if n > 1:
                assert (out2[1].float() == 0).all() and torch.isneginf(lse2[1]).all()
            # exactness: the same as attention over those positions read from the history
            pos = np.full((n, k * P), -1, dtype=np.int32)
            for r in range(n):
                for i in range(k):
                    if S[r, i] >= 0:
                        for o in range(P):
                            if S[r, i] * P + o < lens[r]:
                                pos[r, i * P + o] = S[r, i] * P + o
            o3, _ = oracle.attend_rows(qb, pos, p.orc.host[:, 0], layout, SCALE)
            assert np.abs(out_o2 - o3).max() < 1e-12
    finally:
        p.close()


def test_token_handle_attend_pages_cuts_positions():
    """With page_tokens = 1, hs_attend_pages keeps selected positions below the length."""
    n, k, B, heads = 3, 64, 128, 16
    say("attend_pages on a token handle")
    rng = np.random.default_rng(3)
    p = Pair(n, 1, k, B, 4, hsa.LAYOUT_BF16, seed=8, heads=heads)
    try:
        S = _page_trace(rng, n, 4 * B, k, 0.1)
        slots, _ = p.step(0, S, check_state=False)
        lens = np.array([4 * B, 200, 1], dtype=np.int32)
        qb = skv.queries(8, 0, n, 0, heads)
        out, lse = p.hs.attend_pages(0, _q(qb), torch.from_numpy(slots).cuda(), torch.from_numpy(S).cuda(),
                                     torch.from_numpy(lens).cuda(), SCALE)
        idx = np.where((S >= 0) & (S < lens[:, None]), slots, -1)
        out_o, lse_o = p.orc.attend(0, qb, idx, SCALE)
        torch.cuda.synchronize()
        _compare(out, lse, out_o, lse_o, "token handle, cut")
    finally:
        p.close()


def test_page_graph_capture_and_no_io():
    """resolve + attend_pages captured in one graph and replayed per step equals the eager
    oracle chain; a no-IO handle keeps the same tables."""
    w = C.PAGES.with_(n=4, steps=20)
    P = w.page_tokens
    say(f"pages graph: n {w.n}, P {P}, k {w.k}, B {w.B}, 20 steps")
    x = trace_for(w)
    p = Pair(w.n, 1, w.k, w.B, w.ratio, w.layout, w.seed, heads=16, page_tokens=P)
    noio = hsa.HiSparse(w.k, w.B, w.ratio, w.n, 1, w.layout, flags=hsa.FLAG_NO_IO, page_tokens=P)
    sel = torch.empty(w.n, w.k, dtype=torch.int32, device="cuda")
    lens = torch.empty(w.n, dtype=torch.int32, device="cuda")
    q = torch.empty(w.n, 16, 576, dtype=torch.bfloat16, device="cuda")
    slots = torch.empty_like(sel)
    miss = torch.empty(w.n, dtype=torch.int32, device="cuda")
    out = torch.empty(w.n, 16, 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(w.n, 16, dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    try:
        g = torch.cuda.CUDAGraph()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                p.hs.resolve(0, sel, slots, miss, stream=stream)
                p.hs.attend_pages(0, q, slots, sel, lens, SCALE, out, lse, stream=stream)
        torch.cuda.synchronize()
        for t in range(x.shape[0]):
            L = np.full(w.n, w.len_tokens(t), dtype=np.int32)
            qb = skv.queries(w.seed, t, w.n, 0, 16)
            sel.copy_(torch.from_numpy(x[t]))
            lens.copy_(torch.from_numpy(L))
            q.copy_(_q(qb))
            torch.cuda.synchronize()
            with torch.cuda.stream(stream):
                g.replay()
            s2, m2 = noio.resolve(0, sel)
            torch.cuda.synchronize()
            slots_o, miss_o = p.orc.resolve(0, x[t])
            assert (slots.cpu().numpy() == slots_o).all() and (miss.cpu().numpy() == miss_o).all()
            assert (s2.cpu().numpy() == slots_o).all() and (m2.cpu().numpy() == miss_o).all()
            if t % 5 == 4:
                p.check_state(0, w.n)
                out_o, lse_o = p.orc.attend_pages(0, qb, slots_o, x[t], L, SCALE)
                _compare(out, lse, out_o, lse_o, f"step {t}")
    finally:
        p.close()
        noio.close()


def test_page_workload_full_size_sampled():
    """The page workload at full size (256 requests, pages of 16, 128 pages selected, 256
    slots): tables exact every step; resident bytes and attention sampled."""
    w = C.PAGES
    P = w.page_tokens
    steps = 18
    say(f"pages full size: n {w.n}, P {P}, k {w.k}, B {w.B}, {steps} steps")
    x = trace_for(w, steps=steps)
    p = Pair(w.n, 1, w.k, w.B, w.ratio, w.layout, w.seed, heads=16, oracle_rows=False, page_tokens=P)
    try:
        for t in range(steps):
            slots, _ = p.step(0, x[t], check_state=False)
            if t in (0, 9, steps - 1):
                p.check_state(0, w.n, sample_rows=8)
                L = np.full(w.n, w.len_tokens(t), dtype=np.int32)
                qb = skv.queries(w.seed, t, w.n, 0, 16)
                out, lse = p.hs.attend_pages(0, _q(qb), torch.from_numpy(slots).cuda(),
                                             torch.from_numpy(x[t]).cuda(), torch.from_numpy(L).cuda(), SCALE)
                torch.cuda.synchronize()
                # sampled requests against attention over positions read from the history
                for r in (0, 77, w.n - 1):
                    pos = np.full((1, w.k * P), -1, dtype=np.int32)
                    for i in range(w.k):
                        for o in range(P):
                            if x[t, r, i] * P + o < L[r]:
                                pos[0, i * P + o] = x[t, r, i] * P + o
                    valid = pos[pos >= 0]
                    rows = skv.rows_at(w.seed, r, 0, valid, w.layout)
                    idx = np.full_like(pos, -1)
                    idx[pos >= 0] = np.arange(valid.size)
                    out_o, lse_o = oracle.attend_rows(qb[r:r + 1], idx, rows[None], w.layout, SCALE)
                    err = _compare(out[r:r + 1], lse[r:r + 1], out_o, lse_o, f"step {t} request {r}")
                    say(f"step {t} request {r}: max abs error {err:.3e}")
    finally:
        p.close()


@pytest.mark.parametrize("policy", [hsa.EVICT_LRU, hsa.EVICT_RANDOM])
def test_page_append_writes_through(policy):
    """Page-mode append against the oracle: rows land in the history and in resident pages'
    slots, tables stay, pages brought in later carry the new rows, out-of-range positions flag."""
    P, n, B, k, ratio = 8, 3, 24, 10, 5
    say(f"pages append: P {P}, n {n}, B {B}, k {k}, policy {policy}")
    rng = np.random.default_rng(70 + policy)
    p = Pair(n, 1, k, B, ratio, hsa.LAYOUT_FP8, seed=19, policy=policy, policy_seed=4, page_tokens=P)
    cap_tok = ratio * B * P
    try:
        for t in range(12):
            pos = rng.integers(0, cap_tok, size=n).astype(np.int32)
            if t % 3 == 0:
                pos[0] = -1
            sel = _page_trace(rng, n, ratio * B, k, 0.0)
            for r in range(n):                    # half the time the new token's page is selected
                if pos[r] >= 0 and rng.random() < 0.5 and pos[r] // P not in sel[r]:
                    sel[r, 0] = pos[r] // P
            rows = rng.integers(0, 256, size=(n, 656), dtype=np.uint8)
            s_o = p.orc.append(0, pos, rows)
            s_d = p.hs.append(0, torch.from_numpy(pos).cuda(), torch.from_numpy(rows).cuda())
            torch.cuda.synchronize()
            assert (s_d.cpu().numpy() == s_o).all(), f"step {t}: append slots"
            for r in range(n):
                assert (p.hs.host_kv(0, r) == p.orc.host[r, 0]).all(), f"step {t}: history rows"
            p.check_state(0, n)                   # tables unchanged and slot bytes equal the oracle's
            p.step(0, sel, check_state=True)
        bad = np.array([cap_tok, -1, -1], dtype=np.int32)
        s_d = p.hs.append(0, torch.from_numpy(bad).cuda(), torch.zeros(n, 656, dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
        assert (s_d.cpu().numpy() == -1).all()
        assert p.hs.device_error() & hsa.DEVERR_TOKEN_RANGE
        p.check_state(0, n)
    finally:
        p.close()


def test_page_offload_is_per_token():
    P, n, B, k = 8, 2, 16, 4
    hs = hsa.HiSparse(k, B, 4, n, 1, hsa.LAYOUT_FP8, num_heads=16, page_tokens=P)
    try:
        assert hs.host_kv(0, 1).shape == (4 * B * P, 656)
        rows = torch.from_numpy(skv.rows_at(2, 1, 0, np.arange(4 * B * P), hsa.LAYOUT_FP8)).cuda()
        hs.offload(0, 1, 0, rows)
        with pytest.raises(hsa.HSError):
            hs.offload(0, 1, 4 * B * P - 3, rows[:4])
        torch.cuda.synchronize()
        assert (hs.host_kv(0, 1) == rows.cpu().numpy()).all()
        S = torch.tensor([[-1, -1, -1, -1], [3, 0, -1, 60]], dtype=torch.int32, device="cuda")
        slots, miss = hs.resolve(0, S)
        torch.cuda.synchronize()
        buf = hs.state(0)["kv_buffer"][1].cpu().numpy()
        for i, c in enumerate([3, 0, -1, 60]):
            if c >= 0:
                j = int(slots[1, i])
                assert (buf[j] == rows[c * P:(c + 1) * P].cpu().numpy().reshape(-1)).all()
        assert int(miss[0]) == 0 and int(miss[1]) == 3
    finally:
        hs.close()
