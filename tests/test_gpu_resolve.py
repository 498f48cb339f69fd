"""Resolver parity on the GPU: bit-exact page table, slot owners, stamps, step counters,
output slots, miss counts and slot bytes against the CPU oracle, on the seeded workloads
and on edge cases (padding, ragged sizes, B = k, k = 1, invalid input, no-IO mode,
reset, graph capture)."""
import ctypes

import numpy as np
import pytest
import torch

import hierarchical_kv_cache_hs_amd as hsa
from synth import configs as C
from synth import kv as skv

from gpu_harness import Pair, say, trace_for, fill_host_pool

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]


def _run(w, steps=None, requests=None, check_every=1, oracle_rows=True, sample_rows=None, split=False,
         rows_every=None):
    """Every step: output slots and miss counts bit-exact.  Every check_every steps (and the
    last): page table, owners, stamps, step counters and the LRU order; slot bytes too, on
    every occupied slot or on sample_rows per request, every rows_every steps (default: with
    the tables)."""
    x = trace_for(w, steps=steps, requests=requests)
    n = x.shape[1]
    p = Pair(n, 1, w.k, w.B, w.ratio, w.layout, w.seed, oracle_rows=oracle_rows, split=split)
    rows_every = rows_every or check_every
    misses = []
    try:
        for t in range(x.shape[0]):
            last = t == x.shape[0] - 1
            _, m = p.step(0, x[t], check_state=False)
            if t % check_every == 0 or last:
                p.check_state(0, n, rows=(t % rows_every == 0 or last), sample_rows=sample_rows)
            if t % 50 == 0:
                say(f"{w.name}: step {t} of {x.shape[0]} matches")
            misses.append(m)
    finally:
        p.close()
    return np.stack(misses)


@pytest.mark.parametrize("mode", ["fused", "split"])
def test_tiny_all_steps(mode):
    say(f"tiny: 1 request, k 64, B 128, 32 steps, {mode}")
    m = _run(C.TINY, split=(mode == "split"))
    assert m[0, 0] == 64 and m[1:].max() <= 64


@pytest.mark.parametrize("mode", ["fused", "split"])
def test_batch64_full(mode):
    say(f"batch64: 64 requests, k 2048, B 4096, cap 32768, 200 steps, {mode}")
    m = _run(C.BATCH64, check_every=20, split=(mode == "split"))
    assert (m[0] == 2048).all()


@pytest.mark.parametrize("B", C.SWEEP_BUFFERS)
def test_sweep_buffers_full_size(B):
    """All 100 steps of the 131072-token buffer sweep: slots and misses every step, tables
    every 10 steps, slot bytes on 256 sampled slots per request (regenerated rows)."""
    w = C.sweep_point(B)
    say(f"sweep: 32 requests, ctx 131072, k 2048, B {B}, cap {w.cap}, all {w.steps} steps")
    m = _run(w, check_every=10, oracle_rows=False, sample_rows=256)
    assert m.shape[0] == 100 and (m[0] == 2048).all()


def test_fp8_256_resolve_all_steps_all_rows():
    """The 256-request fp8 workload at 10 % churn over all 200 steps: slots and misses every
    step, tables every 10 steps, and every occupied slot's bytes against the oracle's copy of
    the device buffer every 50 steps and at the last."""
    w = C.churn_point(0.10)
    say(f"fp8_256 resolve: 256 requests, fp8 656 B, churn 0.1, all {w.steps} steps, all slot rows")
    _run(w, check_every=10, rows_every=50)


@pytest.mark.parametrize("churn", (0.02, 0.30))
def test_fp8_256_resolve_other_churns(churn):
    w = C.churn_point(churn)
    say(f"fp8_256 resolve: 256 requests, fp8 656 B, churn {churn}, 25 steps")
    _run(w, steps=25, check_every=8, oracle_rows=False, sample_rows=128)


@pytest.mark.parametrize("k,B,ratio,n,split", [(700, 1000, 3, 3, False), (1, 7, 5, 2, False), (33, 33, 4, 5, False),
                                                (512, 512, 2, 1, False), (513, 777, 9, 4, False),
                                                (2048, 2048, 3, 2, False), (4096, 6000, 2, 2, False),
                                                (700, 1000, 3, 3, True), (1, 7, 5, 2, True), (4096, 6000, 2, 2, True)])
def test_ragged_shapes_random_traces(k, B, ratio, n, split):
    say(f"ragged: k {k}, B {B}, ratio {ratio}, n {n}, split {split}")
    cap = B * ratio
    rng = np.random.default_rng(k * 7 + B)
    p = Pair(n, 1, k, B, ratio, hsa.LAYOUT_BF16, seed=77, split=split)
    try:
        pop = rng.permutation(cap)
        w = 1.0 / np.arange(1, cap + 1) ** 0.9
        w /= w.sum()
        for t in range(12):
            S = np.stack([rng.choice(pop, k, replace=False, p=w) for _ in range(n)]).astype(np.int32)
            S[rng.random(S.shape) < 0.05] = -1
            if t == 5:
                S[0] = -1          # a row of padding only
            p.step(0, S, check_state=True)
    finally:
        p.close()


@pytest.mark.parametrize("split", [False, True])
def test_maximum_sizes_with_attention(split):
    """The largest selection and buffer the library accepts (top_k 8192, 16384 slots): the
    widest register tiling of the 1024-thread resolver, with hits, misses, evictions and
    padding over 5 steps, and attention over 8192 tokens (16 splits) against the oracle."""
    k, B, ratio, n, heads = 8192, 16384, 2, 2, 16
    say(f"maximum sizes: k {k}, B {B}, ratio {ratio}, n {n}, split {split}, attention on the last step")
    cap = B * ratio
    rng = np.random.default_rng(8192 + split)
    p = Pair(n, 1, k, B, ratio, hsa.LAYOUT_BF16, seed=81, heads=heads, split=split)
    try:
        prev = None
        for t in range(5):
            rows = []
            for r in range(n):
                if prev is None:
                    rows.append(rng.choice(cap, k, replace=False))
                else:
                    keep = prev[r][rng.random(k) < 0.6]
                    keep = keep[keep >= 0]
                    pool = np.setdiff1d(np.arange(cap), keep)
                    rows.append(np.concatenate([keep, rng.choice(pool, k - keep.size, replace=False)]))
            S = np.stack(rows).astype(np.int32)
            prev = S.copy()
            S[rng.random(S.shape) < 0.03] = -1
            slots, m = p.step(0, S, check_state=(t % 2 == 0 or t == 4))
            say(f"step {t}: misses {m.tolist()}")
        qb = skv.queries(81, 4, n, 0, heads)
        q = torch.from_numpy(qb.view(np.int16)).cuda().view(torch.bfloat16)
        out, lse = p.hs.attend(0, q, torch.from_numpy(slots).cuda(), 1.0 / 24.0)
        torch.cuda.synchronize()
        out_o, lse_o = p.orc.attend(0, qb, slots, 1.0 / 24.0)
        err = np.abs(out.float().cpu().numpy().astype(np.float64) - out_o).max()
        lerr = np.abs(lse.cpu().numpy().astype(np.float64) - lse_o).max()
        say(f"attention max abs error {err:.3e}, lse {lerr:.3e}")
        assert err <= 2e-2 and lerr <= 1e-3
    finally:
        p.close()


def test_widest_tiling_of_the_512_thread_resolver():
    """More than 128 requests copying rows take the 512-thread resolver; with 16384 slots it
    holds 32 LRU-order entries per thread (its widest tiling)."""
    k, B, ratio, n = 64, 16384, 2, 130
    say(f"512-thread resolver: k {k}, B {B}, n {n}, fp8 rows, 4 steps")
    cap = B * ratio
    rng = np.random.default_rng(130)
    p = Pair(n, 1, k, B, ratio, hsa.LAYOUT_FP8, seed=13)
    try:
        for t in range(4):
            S = np.stack([rng.choice(cap if t < 2 else 96, k, replace=False) for _ in range(n)]).astype(np.int32)
            S[rng.random(S.shape) < 0.05] = -1
            p.step(0, S, check_state=False)
        p.check_state(0, n, sample_rows=32)
    finally:
        p.close()


def test_fewer_requests_than_slots_and_layers_independent():
    say("n_req < max_requests, two layers")
    p = Pair(6, 2, 64, 128, 4, hsa.LAYOUT_FP8, seed=5)
    rng = np.random.default_rng(0)
    try:
        for t in range(10):
            nr = 1 + t % 6
            for layer in (0, 1):
                S = np.stack([rng.choice(512, 64, replace=False) for _ in range(nr)]).astype(np.int32)
                p.step(layer, S, check_state=False)
                p.check_state(layer, 6)
    finally:
        p.close()


def test_injected_host_allocation_failure(monkeypatch):
    """HS_FAULT_INJECT=host_alloc makes the pinned host allocation fail inside hs_create after
    the library allocated its own device block: HS_ERR_OUT_OF_MEMORY, no handle, the device
    block freed again (device memory back where it was after three attempts), and a handle
    created afterwards resolves bit-exactly against the oracle."""
    say("fault injection: pinned host allocation failure in hs_create")
    cfg = hsa.make_config(2048, 4096, 8, 64, 1, hsa.LAYOUT_BF16)    # device_mem NULL: library-owned block
    need = hsa.device_bytes(cfg)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    monkeypatch.setenv("HS_FAULT_INJECT", "host_alloc")
    h = ctypes.c_void_p()
    for _ in range(3):
        st = hsa.lib().hs_create(ctypes.byref(cfg), ctypes.byref(h))
        assert st == hsa.HS_ERR_OUT_OF_MEMORY and not h.value
        assert "injected" in hsa.lib().hs_last_error_message().decode()
    free1 = torch.cuda.mem_get_info()[0]
    assert abs(free0 - free1) < need // 2, f"device memory {free0 - free1} bytes lower after failed creations"
    monkeypatch.delenv("HS_FAULT_INJECT")
    rng = np.random.default_rng(55)
    p = Pair(3, 1, 64, 128, 4, hsa.LAYOUT_BF16, seed=55)
    try:
        for t in range(6):
            p.step(0, np.stack([rng.choice(512, 64, replace=False) for _ in range(3)]).astype(np.int32),
                   check_state=True)
    finally:
        p.close()


def test_invalid_entries_flagged_and_skipped():
    say("invalid tokens: out of range and duplicates")
    hs = hsa.HiSparse(top_k=8, device_buffer_size=16, host_to_device_ratio=4, max_requests=2)
    try:
        fill_host_pool(hs, 3)
        assert hs.device_error() == 0
        sel = torch.tensor([[1, 2, 64, -5, 3, -1, 4, 5], [1, 2, 3, 4, 5, 6, 7, 8]], dtype=torch.int32).cuda()
        slots, miss = hs.resolve(0, sel)
        s = slots.cpu().numpy()
        assert hs.device_error() == hsa.DEVERR_TOKEN_RANGE
        assert s[0, 2] == -1 and s[0, 3] == -1 and s[0, 5] == -1
        assert miss.cpu().numpy().tolist() == [5, 8]
        sel = torch.tensor([[9, 9, 1, 2, 3, 4, 5, 6], [1, 1, 1, 1, 1, 1, 1, 1]], dtype=torch.int32).cuda()
        slots, miss = hs.resolve(0, sel)
        s = slots.cpu().numpy()
        assert hs.device_error() == hsa.DEVERR_DUPLICATE
        assert sorted([s[0, 0], s[0, 1]])[0] == -1 and max(s[0, 0], s[0, 1]) >= 0
        assert (s[1] >= 0).sum() == 1
        st = hs.state(0)
        pt = st["page_table"].cpu().numpy()
        rm = st["slot_owner"].cpu().numpy()
        for r in range(2):
            res = np.nonzero(pt[r] >= 0)[0]
            assert all(rm[r, pt[r, x]] == x for x in res)
        assert hs.device_error() == 0
    finally:
        hs.close()


def test_no_io_mode_same_tables_no_rows():
    say("no-IO mode")
    w = C.TINY.with_(n=3)
    x = trace_for(w)
    a = hsa.HiSparse(64, 128, 32, 3)
    b = hsa.HiSparse(64, 128, 32, 3, flags=hsa.FLAG_NO_IO)
    try:
        fill_host_pool(a, w.seed)
        with pytest.raises(hsa.HSError):          # no host pool in no-IO mode
            b.host_kv_ptr(0, 0)
        b.state(0)["kv_buffer"].zero_()
        for t in range(x.shape[0]):
            sel = torch.from_numpy(x[t]).cuda()
            sa, ma = a.resolve(0, sel)
            sb, mb = b.resolve(0, sel)
            assert torch.equal(sa, sb) and torch.equal(ma, mb)
        A, Bs = a.state(0), b.state(0)
        for key in ("page_table", "slot_owner", "slot_stamp", "lru_order", "step"):
            assert torch.equal(A[key], Bs[key]), key
        assert not bool(Bs["kv_buffer"].any())
    finally:
        a.close()
        b.close()


def test_reset_requests_restores_empty_state():
    say("reset_requests")
    p = Pair(4, 2, 64, 128, 8, hsa.LAYOUT_BF16, seed=9)
    rng = np.random.default_rng(1)
    try:
        for t in range(5):
            for layer in (0, 1):
                S = np.stack([rng.choice(1024, 64, replace=False) for _ in range(4)]).astype(np.int32)
                p.step(layer, S, check_state=False)
        p.hs.reset_requests(1, 2)
        torch.cuda.synchronize()
        for layer in (0, 1):
            st = p.hs.state(layer)
            assert (st["page_table"][1:3] == -1).all() and (st["slot_owner"][1:3] == -1).all()
            assert (st["slot_stamp"][1:3] == -1).all() and (st["step"][1:3] == 0).all()
            assert torch.equal(st["lru_order"][1:3].cpu(), torch.arange(128, dtype=torch.int32).repeat(2, 1))
            assert (st["step"][0] == 5) and (st["step"][3] == 5)
    finally:
        p.close()


def test_deterministic_repeat():
    say("determinism: two handles, same trace")
    w = C.BATCH64.with_(n=8, steps=20)
    x = trace_for(w)
    outs = []
    for _ in range(2):
        hs = hsa.HiSparse(2048, 4096, 8, 8)
        fill_host_pool(hs, w.seed)
        res = []
        for t in range(x.shape[0]):
            s, m = hs.resolve(0, torch.from_numpy(x[t]).cuda())
            res.append((s.cpu(), m.cpu()))
        st = hs.state(0)
        res.append(tuple(st[k].cpu() for k in ("page_table", "slot_owner", "slot_stamp", "lru_order")))
        res.append(st["kv_buffer"].cpu())
        outs.append(res)
        hs.close()
    for a, b in zip(*outs):
        if isinstance(a, tuple):
            assert all(torch.equal(u, v) for u, v in zip(a, b))
        else:
            assert torch.equal(a, b)


def test_graph_capture_replays_match_eager():
    say("hipGraph capture of resolve, replayed over a trace")
    w = C.BATCH64.with_(n=4, steps=12)
    x = trace_for(w)
    eager = hsa.HiSparse(2048, 4096, 8, 4)
    graphed = hsa.HiSparse(2048, 4096, 8, 4)
    try:
        for h in (eager, graphed):
            fill_host_pool(h, w.seed)
        sel = torch.from_numpy(x[0]).cuda()
        slots = torch.empty_like(sel)
        miss = torch.empty(4, dtype=torch.int32, device="cuda")
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                graphed.resolve(0, sel, slots, miss, stream=s)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        # capture did not run the kernel: tables are still empty
        assert int(graphed.state(0)["step"].sum()) == 0
        for t in range(x.shape[0]):
            sel.copy_(torch.from_numpy(x[t]))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            es, em = eager.resolve(0, torch.from_numpy(x[t]).cuda())
            torch.cuda.synchronize()
            assert torch.equal(es, slots) and torch.equal(em, miss), f"replay {t}"
        A, Bs = eager.state(0), graphed.state(0)
        for key in ("page_table", "slot_owner", "slot_stamp", "lru_order", "step", "kv_buffer"):
            assert torch.equal(A[key], Bs[key]), key
    finally:
        eager.close()
        graphed.close()


def test_empty_batches_are_accepted_and_change_nothing():
    """Every enqueueing entry point with zero requests returns success, launches nothing and
    leaves the tables, the device buffer and the error word as they were (between two steps of
    a real trace, so the state is not empty)."""
    w = C.TINY.with_(n=3)
    x = trace_for(w, steps=4)
    p = Pair(w.n, 1, w.k, w.B, w.ratio, w.layout, w.seed, heads=16)
    try:
        for t in range(2):
            p.step(0, x[t], check_state=False)
        hs = p.hs
        torch.cuda.synchronize()
        before = {k: v.clone() for k, v in hs.state(0).items() if isinstance(v, torch.Tensor)}
        dev = "cuda"
        sel0 = torch.empty(0, w.k, dtype=torch.int32, device=dev)
        q0 = torch.empty(0, 16, 576, dtype=torch.bfloat16, device=dev)
        lens0 = torch.empty(0, dtype=torch.int32, device=dev)
        slots, miss = hs.resolve(0, sel0)
        assert slots.shape == (0, w.k) and miss.shape == (0,)
        hs.resolve(0, sel0, split=True)
        hs.resolve_tables(0, sel0, torch.empty(0, w.k, dtype=torch.int32, device=dev),
                          torch.empty(0, dtype=torch.int32, device=dev))
        hs.fetch_misses(0, 0)
        out, lse = hs.attend(0, q0, sel0, 0.1)
        assert out.shape == (0, 16, 512) and lse.shape == (0, 16)
        hs.attend_noalloc(0, q0, sel0, 0.1)
        hs.attend_pages(0, q0, sel0, sel0, lens0, 0.1)
        hs.append(0, torch.empty(0, dtype=torch.int32, device=dev),
                  torch.empty(0, w.entry_bytes, dtype=torch.uint8, device=dev))
        assert hs.topk(torch.empty(0, 64, dtype=torch.float32, device=dev), lens0).shape == (0, w.k)
        torch.cuda.synchronize()
        after = hs.state(0)
        for k, v in before.items():
            assert torch.equal(v, after[k]), f"{k} changed"
        assert hs.device_error() == 0
        # and the trace continues as if nothing had happened
        for t in range(2, 4):
            p.step(0, x[t], check_state=True)
    finally:
        p.close()
