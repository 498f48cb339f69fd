"""Checkpoint and resume through the state views: the tables, the fresh-slot bits, the slot
buffer and the host rows (with the resident-tail layout also the tail plane), exported from one
handle between steps and copied into a fresh handle of the same configuration, continue the run
exactly -- every later slot, miss count, attention output and table equals the uninterrupted
run's, bit for bit."""
import math

import numpy as np
import pytest
import torch

import hierarchical_kv_cache_hs_amd as hsa
from synth import configs as C
from synth import kv as skv
from synth import trace as tr

from gpu_harness import fill_host_pool, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

KEYS = ("page_table", "slot_owner", "slot_stamp", "lru_order", "step", "fresh_slots", "kv_buffer")
SCALE = 1.0 / math.sqrt(576)


def _keys(hs):
    return KEYS + (("tail_plane",) if hs.tail_bytes else ())


def _export(hs):
    dev = [{key: hs.state(l)[key].clone() for key in _keys(hs)} for l in range(hs.L)]
    host = [[hs.host_kv(l, r).copy() for r in range(hs.n)] for l in range(hs.L)]
    return dev, host


def _import(hs, snap):
    dev, host = snap
    for l in range(hs.L):
        st = hs.state(l)
        for key in _keys(hs):
            st[key].copy_(dev[l][key])
        for r in range(hs.n):
            np.copyto(hs.host_kv(l, r), host[l][r])
    torch.cuda.synchronize()


def _same_state(a, b):
    for l in range(a.L):
        sa, sb = a.state(l), b.state(l)
        for key in _keys(a):
            assert torch.equal(sa[key], sb[key]), f"layer {l}: {key} differs"
        for r in range(a.n):
            assert np.array_equal(a.host_kv(l, r), b.host_kv(l, r)), f"layer {l} request {r}: host rows differ"


@pytest.mark.parametrize("policy,flags", [(hsa.EVICT_LRU, 0), (hsa.EVICT_FIFO, 0),
                                          (hsa.EVICT_LRU, hsa.FLAG_RESIDENT_TAIL)])
def test_resume_with_appends_and_attention(policy, flags):
    w = C.FP8_256.with_(n=6, k=256, B=512, ratio=8, steps=14, ctx=3000, window=32)
    L, s = 2, 6
    say(f"resume: policy {policy}, flags {flags}, n {w.n}, layers {L}, k {w.k}, B {w.B}, export at step {s}")
    x = tr.generate(w.trace_spec())
    a = hsa.HiSparse(w.k, w.B, w.ratio, w.n, L, w.layout, 16, flags, eviction=policy)
    b = hsa.HiSparse(w.k, w.B, w.ratio, w.n, L, w.layout, 16, flags, eviction=policy)
    try:
        fill_host_pool(a, w.seed)
        fill_host_pool(b, w.seed + 1)                      # different rows until the import

        def step(hs, t):
            outs = []
            pos = torch.full((w.n,), w.ctx + t, dtype=torch.int32, device="cuda")
            for l in range(L):
                rows = torch.from_numpy(skv.rows_at(99, 0, l, np.arange(w.n) + 7 * t, w.layout)).cuda()
                hs.append(l, pos, rows)
                sel = torch.from_numpy(x[t]).cuda()
                slots, miss = hs.resolve(l, sel)
                q = torch.from_numpy(skv.queries(w.seed, t, w.n, l, 16).view(np.int16)).cuda().view(torch.bfloat16)
                out, lse = hs.attend(l, q, slots, SCALE)
                outs.append((slots, miss, out, lse))
            torch.cuda.synchronize()
            return outs

        for t in range(s):
            step(a, t)
        _import(b, _export(a))
        _same_state(a, b)
        for t in range(s, w.steps):
            ra, rb = step(a, t), step(b, t)
            for l in range(L):
                for va, vb in zip(ra[l], rb[l]):
                    assert torch.equal(va, vb), f"step {t} layer {l}: resumed run differs"
        _same_state(a, b)
        assert a.device_error() == 0 and b.device_error() == 0
    finally:
        a.close()
        b.close()


def test_resume_pages_split_resolve():
    w = C.PAGES.with_(n=5, steps=30)
    s = 11
    P = w.page_tokens
    say(f"resume pages: n {w.n}, P {P}, export at step {s}")
    x = tr.generate(w.trace_spec())
    a = hsa.HiSparse(w.k, w.B, w.ratio, w.n, 1, w.layout, 16, page_tokens=P)
    b = hsa.HiSparse(w.k, w.B, w.ratio, w.n, 1, w.layout, 16, page_tokens=P)
    try:
        fill_host_pool(a, w.seed)

        def step(hs, t):
            sel = torch.from_numpy(x[t]).cuda()
            slots, miss = hs.resolve(0, sel, split=True)
            lens = torch.full((w.n,), w.len_tokens(t), dtype=torch.int32, device="cuda")
            q = torch.from_numpy(skv.queries(w.seed, t, w.n, 0, 16).view(np.int16)).cuda().view(torch.bfloat16)
            out, lse = hs.attend_pages(0, q, slots, sel, lens, SCALE)
            torch.cuda.synchronize()
            return slots, miss, out, lse

        for t in range(s):
            step(a, t)
        _import(b, _export(a))
        for t in range(s, w.steps):
            for va, vb in zip(step(a, t), step(b, t)):
                assert torch.equal(va, vb), f"step {t}: resumed run differs"
        _same_state(a, b)
    finally:
        a.close()
        b.close()
