"""Write-through append and prefill offload on the GPU, through the C ABI, against the oracle.

Append (hs_append) must leave the same page table, owners, stamps, step counters and slot
bytes as the oracle's append, keep the LRU order array sorted by (stamp, slot), and write
the row to the host history; offload (hs_offload) must put rows at the right history
positions.  All comparisons are bit-exact."""
import numpy as np
import pytest
import torch

import hierarchical_kv_cache_hs_amd as hsa
import oracle
from synth import configs as C
from synth import kv as skv

from gpu_harness import fill_host_pool, history, lru_order_ok, say, trace_for

TAIL = hsa.FLAG_RESIDENT_TAIL

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]


def _check_tables(hs, orc, nr, layer=0, rows=True):
    st = hs.state(layer)
    pt = st["page_table"][:nr].cpu().numpy()
    rm = st["slot_owner"][:nr].cpu().numpy()
    stamp = st["slot_stamp"][:nr].cpu().numpy()
    order = st["lru_order"][:nr].cpu().numpy()
    assert (pt == orc.PT[:nr, layer]).all(), "page table differs"
    assert (rm == orc.RM[:nr, layer]).all(), "slot owners differ"
    assert (stamp.astype(np.int64) == orc.ST[:nr, layer]).all(), "stamps differ"
    assert (st["step"][:nr].cpu().numpy() == orc.t[:nr, layer]).all(), "step counters differ"
    assert lru_order_ok(stamp, order), "LRU order is not (stamp, slot) sorted"
    if rows:
        buf = st["kv_buffer"][:nr].cpu().numpy()
        for r in range(nr):
            occ = np.nonzero(rm[r] >= 0)[0]
            assert (buf[r, occ] == orc.dev[r, layer, occ]).all(), f"slot bytes differ (request {r})"
        assert not bool(st["zero_row"].any()), "zero row written"


@pytest.mark.parametrize("layout,flags", [(hsa.LAYOUT_BF16, 0), (hsa.LAYOUT_FP8, 0), (hsa.LAYOUT_FP8, TAIL)])
def test_append_interleaved_with_resolve_matches_oracle(layout, flags):
    n, B, k, ratio, seed = 3, 64, 24, 4, 77
    cap = ratio * B
    say(f"append vs oracle: layout {layout}, flags {flags}, n {n}, B {B}, k {k}, cap {cap}")
    rng = np.random.default_rng(5)
    hs = hsa.HiSparse(k, B, ratio, n, 1, layout, flags=flags)
    try:
        fill_host_pool(hs, seed)
        E = skv.ENTRY_BYTES[layout]
        host = np.stack([np.stack([history(hs, 0, r)]) for r in range(n)])  # [n][1][cap][E]
        orc = oracle.OracleCache(n, 1, B, cap, layout=layout, host=np.ascontiguousarray(host))
        nxt = np.array([10, 20, 30])
        for step in range(40):
            pos = nxt.copy().astype(np.int32)
            nxt += 1
            pos[rng.random(n) < 0.2] = -1                            # no token for some requests
            re = rng.random(n) < 0.15                                 # or one that may be resident
            pos[re] = rng.integers(0, cap, size=int(re.sum()))
            rows = rng.integers(0, 256, size=(n, E), dtype=np.uint8)
            s_o = orc.append(0, pos, rows)
            s_d = hs.append(0, torch.from_numpy(pos).cuda(), torch.from_numpy(rows).cuda())
            torch.cuda.synchronize()
            assert (s_d.cpu().numpy() == s_o).all(), f"step {step}: append slots differ"
            _check_tables(hs, orc, n)
            S = np.stack([rng.choice(cap, k, replace=False) for _ in range(n)]).astype(np.int32)
            for r in range(n):                                        # most steps select the new token
                if pos[r] >= 0 and rng.random() < 0.8 and pos[r] not in S[r]:
                    S[r, 0] = pos[r]
            slots_d, miss_d = hs.resolve(0, torch.from_numpy(S).cuda())
            slots_o, miss_o = orc.resolve(0, S)
            torch.cuda.synchronize()
            assert (slots_d.cpu().numpy() == slots_o).all() and (miss_d.cpu().numpy() == miss_o).all()
            _check_tables(hs, orc, n)
        for r in range(n):
            assert (history(hs, 0, r) == orc.host[r, 0]).all(), f"host history differs (request {r})"
        assert hs.device_error() == 0
    finally:
        hs.close()


def test_append_sliding_window_has_no_misses():
    # the oracle's closed form on the device: B > k and the newest token appended before
    # each step -> no step misses; the same trace without append misses once per step
    n, k, B = 4, 32, 40
    say(f"append sliding window: n {n}, k {k}, B {B}")
    a = hsa.HiSparse(k, B, 8, n, 1, hsa.LAYOUT_BF16)
    b = hsa.HiSparse(k, B, 8, n, 1, hsa.LAYOUT_BF16)
    try:
        rows = torch.zeros(n, 1152, dtype=torch.uint8, device="cuda")
        for t in range(3 * B):
            S = np.full((n, k), -1, dtype=np.int32)
            win = np.arange(max(0, t - k + 1), t + 1, dtype=np.int32)
            S[:, : win.size] = win
            a.append(0, torch.full((n,), t, dtype=torch.int32, device="cuda"), rows)
            _, ma = a.resolve(0, torch.from_numpy(S).cuda())
            _, mb = b.resolve(0, torch.from_numpy(S).cuda())
            torch.cuda.synchronize()
            assert (ma.cpu() == 0).all(), f"step {t}: misses with append"
            assert (mb.cpu() == 1).all(), f"step {t}: expected one miss without append"
    finally:
        a.close()
        b.close()


def test_append_out_of_range_sets_error_and_changes_nothing():
    n, B, k = 2, 16, 8
    hs = hsa.HiSparse(k, B, 2, n, 1, hsa.LAYOUT_BF16)
    try:
        hs.resolve(0, torch.arange(n * k, dtype=torch.int32, device="cuda").view(n, k) % (2 * B))
        torch.cuda.synchronize()
        before = {key: v.clone() for key, v in hs.state(0).items() if torch.is_tensor(v)}
        pos = torch.tensor([2 * B, -7], dtype=torch.int32, device="cuda")
        out = hs.append(0, pos, torch.ones(n, 1152, dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
        assert (out.cpu() == -1).all()
        assert hs.device_error() & hsa.DEVERR_TOKEN_RANGE
        after = hs.state(0)
        for key, v in before.items():
            assert torch.equal(v, after[key]), key
    finally:
        hs.close()


@pytest.mark.parametrize("flags", [0, TAIL])
def test_append_and_resolve_in_a_graph_replay_like_eager(flags):
    n, B, k, ratio, seed = 4, 128, 48, 4, 9
    cap = ratio * B
    say(f"append + resolve captured in a graph, replayed per step, flags {flags}")
    rng = np.random.default_rng(11)
    hs = hsa.HiSparse(k, B, ratio, n, 1, hsa.LAYOUT_FP8, flags=flags)
    try:
        fill_host_pool(hs, seed)
        host = np.stack([np.stack([history(hs, 0, r)]) for r in range(n)])
        orc = oracle.OracleCache(n, 1, B, cap, layout=hsa.LAYOUT_FP8, host=np.ascontiguousarray(host))
        pos_d = torch.zeros(n, dtype=torch.int32, device="cuda")
        rows_d = torch.zeros(n, 656, dtype=torch.uint8, device="cuda")
        sel_d = torch.zeros(n, k, dtype=torch.int32, device="cuda")
        slots_d = torch.empty(n, k, dtype=torch.int32, device="cuda")
        miss_d = torch.empty(n, dtype=torch.int32, device="cuda")
        aslot_d = torch.empty(n, dtype=torch.int32, device="cuda")
        stream = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                hs.append(0, pos_d, rows_d, aslot_d, stream=stream)
                hs.resolve(0, sel_d, slots_d, miss_d, stream=stream)
        torch.cuda.synchronize()
        hs.reset_requests(0, n)                    # the capture did not run; start clean anyway
        torch.cuda.synchronize()
        for step in range(12):
            pos = (100 + step + 7 * np.arange(n)).astype(np.int32)
            rows = rng.integers(0, 256, size=(n, 656), dtype=np.uint8)
            S = np.stack([rng.choice(cap, k, replace=False) for _ in range(n)]).astype(np.int32)
            for r in range(n):                                        # every step selects the new token
                if pos[r] not in S[r]:
                    S[r, 0] = pos[r]
            pos_d.copy_(torch.from_numpy(pos))
            rows_d.copy_(torch.from_numpy(rows))
            sel_d.copy_(torch.from_numpy(S))
            torch.cuda.synchronize()
            with torch.cuda.stream(stream):
                g.replay()
            torch.cuda.synchronize()
            s_o = orc.append(0, pos, rows)
            slots_o, miss_o = orc.resolve(0, S)
            assert (aslot_d.cpu().numpy() == s_o).all(), f"replay {step}: append slots"
            assert (slots_d.cpu().numpy() == slots_o).all() and (miss_d.cpu().numpy() == miss_o).all()
            _check_tables(hs, orc, n)
    finally:
        hs.close()


# without the tail plane: flat copy, store kernel, 2-D copy; with it: store kernel (0, 48),
# two 2-D copies (5)
@pytest.mark.parametrize("flags", [0, TAIL])
@pytest.mark.parametrize("pad", [0, 48, 5])
def test_offload_writes_history_rows(pad, flags):
    n, B, k, ratio = 2, 64, 16, 8
    cap = ratio * B
    E = 656
    say(f"offload: row stride {E + pad}, flags {flags}")
    rng = np.random.default_rng(3 + pad)
    hs = hsa.HiSparse(k, B, ratio, n, 1, hsa.LAYOUT_FP8, flags=flags)
    try:
        before = history(hs, 0, 1)
        first, count = 37, 300
        rows = rng.integers(0, 256, size=(count, E + pad), dtype=np.uint8)
        hs.offload(0, 1, first, torch.from_numpy(rows).cuda())
        torch.cuda.synchronize()
        after = history(hs, 0, 1)
        if flags:   # request 0's tails (zero, like the whole device block at creation) are untouched
            assert not hs.tail_plane(0)[0].any()
        assert (after[first:first + count] == rows[:, :E]).all()
        assert (after[:first] == before[:first]).all() and (after[first + count:] == before[first + count:]).all()
        # the offloaded rows arrive as misses and land in their slots unchanged
        S = np.full((n, k), -1, dtype=np.int32)
        S[1] = np.arange(first, first + k)
        slots, miss = hs.resolve(0, torch.from_numpy(S).cuda())
        torch.cuda.synchronize()
        assert int(miss[1]) == k
        buf = hs.state(0)["kv_buffer"][1].cpu().numpy()
        assert (buf[slots[1].cpu().numpy()] == rows[:k, :E]).all()
        with pytest.raises(hsa.HSError):
            hs.offload(0, 1, cap - 10, torch.from_numpy(rows[:11]).cuda())
    finally:
        hs.close()


def test_append_full_size_fp8_256_growing_context():
    """The 256-request fp8 workload with its newest token appended before every step: tables
    match the oracle bit for bit and the guaranteed miss of the new token disappears."""
    w = C.FP8_256
    steps = 6
    say(f"append at full size: {w.n} requests, k {w.k}, B {w.B}, {steps} steps")
    x = trace_for(w, steps=steps)
    hs = hsa.HiSparse(w.k, w.B, w.ratio, w.n, 1, w.layout)
    try:
        fill_host_pool(hs, w.seed)
        orc = oracle.OracleCache(w.n, 1, w.B, w.cap, layout=w.layout)
        plain = oracle.OracleCache(w.n, 1, w.B, w.cap, layout=w.layout)
        for t in range(steps):
            newest = np.full(w.n, w.ctx + t - 1, dtype=np.int32)
            assert all(newest[r] in x[t, r] for r in range(w.n))
            rows = np.stack([skv.rows_at(w.seed, r, 0, newest[r:r + 1], w.layout)[0] for r in range(w.n)])
            s_o = orc.append(0, newest, rows)
            s_d = hs.append(0, torch.from_numpy(newest).cuda(), torch.from_numpy(rows).cuda())
            slots_d, miss_d = hs.resolve(0, torch.from_numpy(x[t]).cuda())
            slots_o, miss_o = orc.resolve(0, x[t])
            _, miss_p = plain.resolve(0, x[t])
            torch.cuda.synchronize()
            assert (s_d.cpu().numpy() == s_o).all()
            assert (slots_d.cpu().numpy() == slots_o).all() and (miss_d.cpu().numpy() == miss_o).all()
            say(f"step {t}: misses per request {miss_o.mean():.2f} with append, {miss_p.mean():.2f} without")
            if t > 0:
                assert miss_o.sum() < miss_p.sum()
        _check_tables(hs, orc, w.n, rows=False)
        # sampled slots hold their tokens' rows
        st = hs.state(0)
        rm = st["slot_owner"].cpu().numpy()
        buf = st["kv_buffer"]
        for r in (0, 100, 255):
            occ = np.nonzero(rm[r] >= 0)[0][::97]
            assert (buf[r, occ].cpu().numpy() == skv.rows_at(w.seed, r, 0, rm[r, occ], w.layout)).all()
    finally:
        hs.close()
