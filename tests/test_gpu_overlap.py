"""Attention of the resident tokens while the misses are copied (hs_attend_resident beside
hs_fetch_misses, then hs_attend_fetched) against the fp64 oracle.

The two parts split the valid entries of a step exactly: an entry is a miss iff its slot is
one of the step's victim slots, which the miss list names.  Their merge is attention over the
whole selection, so the oracle's attention of the resolved slots is the expected value, at the
tolerances of the single-launch attention: max abs error 2e-2 on the bf16 output and 1e-3 on
the fp32 lse (rounding of the output and of P to bf16; fp32 accumulation), and 1e-5 on both
in the fp32-output mode (P carried to 2^-27 relative).  Resolution stays bit-exact."""
import math

import numpy as np
import pytest
import torch

import hierarchical_kv_cache_hs_amd as hsa
from hierarchical_kv_cache_hs_amd.decode_step import attend_while_fetching
from synth import configs as C
from synth import kv as skv

from gpu_harness import Pair, say, trace_for

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

SCALE = 1.0 / math.sqrt(576)


def _compare(out_g, lse_g, out_o, lse_o, tol_out, tol_lse, what):
    og = out_g.float().cpu().numpy().astype(np.float64)
    lg = lse_g.cpu().numpy().astype(np.float64)
    err = np.abs(og - out_o).max() if og.size else 0.0
    assert err <= tol_out, f"{what}: max abs error {err}"
    fin = np.isfinite(lse_o)
    assert (np.isfinite(lg) == fin).all(), f"{what}: lse finiteness differs"
    if fin.any():
        lerr = np.abs(lg[fin] - lse_o[fin]).max()
        assert lerr <= tol_lse, f"{what}: lse error {lerr}"
    return err


def _q(qb):
    return torch.from_numpy(qb.view(np.int16)).cuda().view(torch.bfloat16)


def _selection(rng, n, cap, k, prev=None):
    """n distinct-token selections of k from [0, cap); with prev, the first half repeats prev's
    (hits) and the rest are drawn from the other tokens (mostly misses)."""
    rows = []
    for r in range(n):
        if prev is None:
            rows.append(rng.choice(cap, k, replace=False))
            continue
        keep = prev[r, : k // 2]
        pool = np.setdiff1d(np.arange(cap), keep[keep >= 0])
        rows.append(np.concatenate([keep, rng.choice(pool, k - keep.size, replace=False)]))
    return np.stack(rows).astype(np.int32)


class Overlapped:
    """Steps a Pair with the overlapped layer (two streams) and checks every step."""

    def __init__(self, p: Pair, heads: int):
        self.p, self.heads = p, heads
        self.main = torch.cuda.Stream()
        self.side = torch.cuda.Stream()

    def step(self, layer, S, qb, lens=None):
        p, n = self.p, S.shape[0]
        sel = torch.from_numpy(np.ascontiguousarray(S, dtype=np.int32)).cuda()
        q = _q(qb)
        d_lens = None if lens is None else torch.from_numpy(lens).cuda()
        slots = torch.empty_like(sel)
        miss = torch.empty(n, dtype=torch.int32, device="cuda")
        out = torch.empty(n, self.heads, 512, dtype=p.hs.out_dtype, device="cuda")
        lse = torch.empty(n, self.heads, dtype=torch.float32, device="cuda")
        self.main.wait_stream(torch.cuda.current_stream())
        attend_while_fetching(p.hs, layer, sel, q, SCALE, slots, miss, out, lse, self.main, self.side, d_lens)
        torch.cuda.current_stream().wait_stream(self.main)
        torch.cuda.synchronize()
        slots_o, miss_o = p.orc.resolve(layer, S)
        assert (slots.cpu().numpy() == slots_o).all(), "slots differ"
        assert (miss.cpu().numpy() == miss_o).all(), "miss counts differ"
        if lens is None:
            out_o, lse_o = p.orc.attend(layer, qb, slots_o, SCALE)
        else:
            out_o, lse_o = p.orc.attend_pages(layer, qb, slots_o, S, lens, SCALE)
        return out, lse, out_o, lse_o, miss_o


@pytest.mark.parametrize("layout", [hsa.LAYOUT_BF16, hsa.LAYOUT_FP8])
def test_overlap_tiny_every_step(layout):
    w = C.TINY.with_(layout=layout, n=2)
    say(f"overlap tiny, layout {layout}: 2 requests, k 64, B 128, 32 steps")
    x = trace_for(w)
    p = Pair(w.n, 1, w.k, w.B, w.ratio, layout, w.seed, heads=16)
    ov = Overlapped(p, 16)
    worst = 0.0
    try:
        for t in range(x.shape[0]):
            out, lse, out_o, lse_o, miss = ov.step(0, x[t], skv.queries(w.seed, t, w.n, 0, 16))
            worst = max(worst, _compare(out, lse, out_o, lse_o, 2e-2, 1e-3, f"step {t} ({miss.tolist()} misses)"))
        p.check_state(0, w.n)
    finally:
        p.close()
    say(f"worst abs error {worst:.3e}")


@pytest.mark.parametrize("policy", [hsa.EVICT_FIFO, hsa.EVICT_RANDOM])
def test_overlap_under_other_eviction_policies(policy):
    """The miss list names the step's victims under every policy, so the resident part skips
    exactly the slots the copy writes; tiny trace, fp8, every step against the oracle."""
    w = C.TINY.with_(layout=hsa.LAYOUT_FP8, n=3)
    say(f"overlap, eviction policy {policy}: 3 requests, k 64, B 128, 32 steps")
    x = trace_for(w)
    p = Pair(w.n, 1, w.k, w.B, w.ratio, w.layout, w.seed, heads=16, policy=policy, policy_seed=99)
    ov = Overlapped(p, 16)
    try:
        for t in range(x.shape[0]):
            out, lse, out_o, lse_o, _ = ov.step(0, x[t], skv.queries(w.seed, t, w.n, 0, 16))
            _compare(out, lse, out_o, lse_o, 2e-2, 1e-3, f"step {t}")
        p.check_state(0, w.n)
    finally:
        p.close()


@pytest.mark.parametrize("layout,heads,k,B,n", [(hsa.LAYOUT_BF16, 16, 100, 160, 3), (hsa.LAYOUT_FP8, 5, 37, 64, 2),
                                                (hsa.LAYOUT_BF16, 1, 1, 4, 2), (hsa.LAYOUT_FP8, 16, 1000, 1024, 1),
                                                (hsa.LAYOUT_BF16, 16, 2048, 4096, 300)])
def test_overlap_ragged_shapes_and_padding(layout, heads, k, B, n):
    say(f"overlap ragged: layout {layout}, heads {heads}, k {k}, B {B}, n {n}")
    rng = np.random.default_rng(k + heads + 5)
    cap = 4 * B
    p = Pair(n, 1, k, B, 4, layout, seed=37, heads=heads)
    ov = Overlapped(p, heads)
    try:
        prev = None
        for t in range(4):
            S = _selection(rng, n, cap, k, prev if t == 3 else None)   # step 3: hits and misses
            S[rng.random(S.shape) < 0.2] = -1
            if n > 1:
                S[1] = -1       # a request with no valid entry: out 0, lse -inf
            prev = S.copy()
            out, lse, out_o, lse_o, _ = ov.step(0, S, skv.queries(37, t, n, 0, heads))
            _compare(out, lse, out_o, lse_o, 2e-2, 1e-3, f"step {t}")
            if n > 1:
                assert (out[1].float() == 0).all() and torch.isneginf(lse[1]).all()
    finally:
        p.close()


@pytest.mark.parametrize("layout", [hsa.LAYOUT_BF16, hsa.LAYOUT_FP8])
def test_overlap_fp32_output_tier(layout):
    w = C.TINY.with_(layout=layout, n=3)
    say(f"overlap fp32 output, layout {layout}: 3 requests, k 64, B 128, 32 steps, tolerance 1e-5")
    x = trace_for(w)
    p = Pair(w.n, 1, w.k, w.B, w.ratio, layout, w.seed, heads=16, flags=hsa.FLAG_ATTN_OUT_F32)
    ov = Overlapped(p, 16)
    try:
        for t in range(x.shape[0]):
            out, lse, out_o, lse_o, _ = ov.step(0, x[t], skv.queries(w.seed, t, w.n, 0, 16))
            assert out.dtype == torch.float32
            _compare(out, lse, out_o, lse_o, 1e-5, 1e-5, f"step {t}")
    finally:
        p.close()


@pytest.mark.parametrize("layout", [hsa.LAYOUT_BF16, hsa.LAYOUT_FP8])
def test_overlap_pages_cut_at_length(layout):
    P, k, B, n, heads = 16, 20, 40, 3, 16
    say(f"overlap pages: P {P}, k {k}, B {B}, n {n}, layout {layout}, cut at ragged lengths")
    rng = np.random.default_rng(91 + layout)
    cap = 4 * B
    p = Pair(n, 1, k, B, 4, layout, seed=29, heads=heads, page_tokens=P)
    ov = Overlapped(p, heads)
    try:
        prev = None
        for t in range(5):
            S = _selection(rng, n, cap, k, prev)
            S[rng.random(S.shape) < 0.15] = -1
            prev = S.copy()
            lens = rng.integers(1, cap * P + 1, size=n).astype(np.int32)
            valid = S[0][S[0] >= 0]
            if valid.size:
                lens[0] = int(valid.max()) * P + P // 2 + 1     # inside the last selected page
            lens[1] = 0                                           # before every page
            out, lse, out_o, lse_o, _ = ov.step(0, S, skv.queries(29, t, n, 0, heads), lens)
            _compare(out, lse, out_o, lse_o, 2e-2, 1e-3, f"step {t}")
            assert (out[1].float() == 0).all() and torch.isneginf(lse[1]).all()
    finally:
        p.close()


def test_overlap_fp8_256_full_size_sampled_steps():
    w = C.churn_point(0.10)
    steps = 12
    say(f"overlap fp8_256: 256 requests, k 2048, B 4096, {steps} steps, attention checked at 0/5/11")
    x = trace_for(w, steps=steps)
    p = Pair(w.n, 1, w.k, w.B, w.ratio, w.layout, w.seed, heads=16)
    ov = Overlapped(p, 16)
    try:
        for t in range(steps):
            qb = skv.queries(w.seed, t, w.n, 0, 16)
            if t in (0, 5, steps - 1):
                out, lse, out_o, lse_o, miss = ov.step(0, x[t], qb)
                err = _compare(out, lse, out_o, lse_o, 2e-2, 1e-3, f"step {t}")
                say(f"step {t}: {miss.mean():.1f} misses per request, max abs error {err:.3e}")
            else:
                p.step(0, x[t], check_state=False)
        p.check_state(0, w.n, sample_rows=64)
    finally:
        p.close()


def test_overlap_graph_replay_equals_eager():
    """Steps captured with the two-stream fork and join, replayed once, give the eager overlapped
    run's outputs bit for bit (same kernels, same inputs), and the same tables."""
    w = C.TINY.with_(layout=hsa.LAYOUT_FP8, n=4)
    T = 12
    say(f"overlap graph: 4 requests, k 64, B 128, fp8, {T} steps captured on two streams")
    x = trace_for(w, steps=T)
    heads = 16
    eager = Pair(w.n, 1, w.k, w.B, w.ratio, w.layout, w.seed, heads=heads, oracle_rows=False)
    graphed = Pair(w.n, 1, w.k, w.B, w.ratio, w.layout, w.seed, heads=heads, oracle_rows=False)
    try:
        sels = torch.from_numpy(x).cuda()
        qs = torch.stack([_q(skv.queries(w.seed, t, w.n, 0, heads)) for t in range(T)])
        outs = [torch.empty(T, w.n, heads, 512, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
        lses = [torch.empty(T, w.n, heads, dtype=torch.float32, device="cuda") for _ in range(2)]
        slots = [torch.empty(T, w.n, w.k, dtype=torch.int32, device="cuda") for _ in range(2)]
        misses = [torch.empty(T, w.n, dtype=torch.int32, device="cuda") for _ in range(2)]
        main, side = torch.cuda.Stream(), torch.cuda.Stream()
        main.wait_stream(torch.cuda.current_stream())
        for t in range(T):
            attend_while_fetching(eager.hs, 0, sels[t], qs[t], SCALE, slots[0][t], misses[0][t], outs[0][t],
                                  lses[0][t], main, side)
        torch.cuda.current_stream().wait_stream(main)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for t in range(T):
                    attend_while_fetching(graphed.hs, 0, sels[t], qs[t], SCALE, slots[1][t], misses[1][t],
                                          outs[1][t], lses[1][t], cap, side)
        torch.cuda.synchronize()
        with torch.cuda.stream(cap):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(slots[0], slots[1]) and torch.equal(misses[0], misses[1])
        assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
        assert torch.equal(lses[0], lses[1])
        for key in ("page_table", "slot_owner", "slot_stamp", "kv_buffer"):
            assert torch.equal(eager.hs.state(0)[key], graphed.hs.state(0)[key]), key
    finally:
        eager.close()
        graphed.close()


def test_overlap_parts_unsupported_without_io_and_stream_read_runs():
    hs = hsa.HiSparse(top_k=64, device_buffer_size=128, host_to_device_ratio=4, max_requests=2, num_layers=1,
                      layout=hsa.LAYOUT_FP8, num_heads=16, flags=hsa.FLAG_NO_IO)
    try:
        q = torch.zeros(2, 16, 576, dtype=torch.bfloat16, device="cuda")
        slots = torch.full((2, 64), -1, dtype=torch.int32, device="cuda")
        with pytest.raises(hsa.HSError) as e:
            hs.attend_resident(0, q, slots, SCALE)
        assert e.value.status == hsa.HS_ERR_UNSUPPORTED
        with pytest.raises(hsa.HSError) as e:
            hs.attend_fetched(0, q, SCALE)
        assert e.value.status == hsa.HS_ERR_UNSUPPORTED
    finally:
        hs.close()
    # the measurement helper: reads the buffer and leaves the sink alone for ordinary data
    src = torch.ones(1 << 20, dtype=torch.float32, device="cuda")
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    hsa.stream_read(src, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 7


def test_attention_parts_require_the_layers_miss_lists():
    """The copy and the parts refuse to run unless the layer's last resolve-side call was a
    list-only resolve of at least as many requests (a fused resolve, an append or a reset in
    between leaves no lists for this step); the fetched part also needs the resident part's
    partials of the same requests, which a whole attention of the layer overwrites."""
    p = Pair(3, 2, 64, 128, 4, hsa.LAYOUT_FP8, seed=3, heads=16)
    try:
        rng = np.random.default_rng(3)
        S = _selection(rng, 3, 512, 64)
        sel = torch.from_numpy(S).cuda()
        q = _q(skv.queries(3, 0, 3, 0, 16))
        slots = torch.empty_like(sel)
        miss = torch.empty(3, dtype=torch.int32, device="cuda")

        def refused(fn):
            with pytest.raises(hsa.HSError) as e:
                fn()
            assert e.value.status == hsa.HS_ERR_INVALID_ARG

        refused(lambda: p.hs.attend_resident(0, q, slots, SCALE))          # nothing resolved yet
        refused(lambda: p.hs.fetch_misses(0, 3))
        p.hs.resolve(0, sel, slots, miss)                                  # fused: no lists
        refused(lambda: p.hs.attend_resident(0, q, slots, SCALE))
        refused(lambda: p.hs.fetch_misses(0, 3))                           # stale lists would corrupt slots
        p.hs.resolve_tables(0, sel[:2], slots[:2], miss[:2])
        refused(lambda: p.hs.attend_resident(0, q, slots, SCALE))          # 3 requests, lists for 2
        refused(lambda: p.hs.attend_resident(1, q, slots, SCALE))          # other layer
        refused(lambda: p.hs.fetch_misses(0, 3))
        refused(lambda: p.hs.fetch_misses(1, 2))
        p.hs.fetch_misses(0, 2)
        refused(lambda: p.hs.attend_fetched(0, q[:2], SCALE))             # no resident partials yet
        p.hs.attend_resident(0, q[:2], slots[:2], SCALE)
        refused(lambda: p.hs.attend_fetched(0, q[:1], SCALE))             # partials of 2 requests
        p.hs.attend_fetched(0, q[:2], SCALE)
        p.hs.attend(0, q[:2], slots[:2], SCALE)                           # reuses the partial space
        refused(lambda: p.hs.attend_fetched(0, q[:2], SCALE))
        p.hs.attend_resident(0, q[:2], slots[:2], SCALE)
        p.hs.attend_fetched(0, q[:2], SCALE)
        p.hs.reset_requests(0, 3)
        refused(lambda: p.hs.attend_fetched(0, q[:2], SCALE))
        refused(lambda: p.hs.fetch_misses(0, 2))
        torch.cuda.synchronize()
    finally:
        p.close()


@pytest.mark.parametrize("layout", [hsa.LAYOUT_BF16, hsa.LAYOUT_FP8])
def test_overlap_parts_empty_on_cold_and_repeated_steps(layout):
    """Degenerate splits: the first step misses every token (the resident part attends nothing),
    the same selection again hits every token (the fetched part attends nothing, the miss list
    is empty); both equal the oracle's attention over the whole selection."""
    n, k, B, heads = 3, 256, 512, 16
    say(f"overlap degenerate parts, layout {layout}: all misses, then all hits")
    rng = np.random.default_rng(5 + layout)
    p = Pair(n, 1, k, B, 4, layout, seed=41, heads=heads)
    ov = Overlapped(p, heads)
    try:
        S = _selection(rng, n, 4 * B, k)
        S[1, k // 2:] = -1                                  # a half-padded request
        for t, want in ((0, k), (1, 0)):
            out, lse, out_o, lse_o, miss = ov.step(0, S, skv.queries(41, t, n, 0, heads))
            assert miss[0] == want and miss[2] == want, f"step {t}: misses {miss.tolist()}"
            _compare(out, lse, out_o, lse_o, 2e-2, 1e-3, f"step {t}")
    finally:
        p.close()

