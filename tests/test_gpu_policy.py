"""Eviction-policy variants (FIFO, RANDOM) on the GPU against the oracle, bit-exact: page
table, owners, stamps, step counters, output slots, miss counts and slot bytes, on the tiny
workload, ragged random traces, padding, the buffer sweep at full size, and append under FIFO.
The policy study itself (misses per buffer size and policy) is bench.py --workload sweep."""
import numpy as np
import pytest
import torch

import hierarchical_kv_cache_hs_amd as hsa
import oracle
from synth import configs as C
from synth import kv as skv

from gpu_harness import Pair, fill_host_pool, say, trace_for

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

POLICIES = [(hsa.EVICT_FIFO, "fifo"), (hsa.EVICT_RANDOM, "random")]


@pytest.mark.parametrize("policy,name", POLICIES)
@pytest.mark.parametrize("split", [False, True])
def test_tiny_every_step(policy, name, split):
    w = C.TINY.with_(n=3)
    say(f"policy {name}: tiny, 3 requests, 32 steps, split {split}")
    x = trace_for(w)
    p = Pair(w.n, 1, w.k, w.B, w.ratio, w.layout, w.seed, split=split, policy=policy, policy_seed=2024)
    try:
        for t in range(x.shape[0]):
            p.step(0, x[t], check_state=True)
    finally:
        p.close()


@pytest.mark.parametrize("policy,name", POLICIES)
@pytest.mark.parametrize("k,B,ratio,n", [(700, 1000, 3, 3), (1, 7, 5, 2), (33, 33, 4, 5), (513, 777, 9, 4),
                                         (4096, 6000, 2, 2), (100, 16384, 2, 1)])
def test_ragged_random_traces(policy, name, k, B, ratio, n):
    say(f"policy {name}: ragged k {k}, B {B}, ratio {ratio}, n {n}")
    cap = B * ratio
    rng = np.random.default_rng(k * 3 + B + policy)
    p = Pair(n, 1, k, B, ratio, hsa.LAYOUT_BF16, seed=5, policy=policy, policy_seed=k + B)
    try:
        pop = rng.permutation(cap)
        wts = 1.0 / np.arange(1, cap + 1) ** 0.9
        wts /= wts.sum()
        for t in range(10):
            S = np.stack([rng.choice(pop, k, replace=False, p=wts) for _ in range(n)]).astype(np.int32)
            S[rng.random(S.shape) < 0.05] = -1
            p.step(0, S, check_state=True)
    finally:
        p.close()


@pytest.mark.parametrize("policy,name", POLICIES)
def test_sweep_full_size(policy, name):
    # the study's own workload: 32 requests, ctx 131072, B 4096, sampled states and rows
    w = C.sweep_point(4096)
    say(f"policy {name}: sweep, 32 requests, ctx 131072, k 2048, B 4096, 24 steps")
    x = trace_for(w, steps=24)
    p = Pair(w.n, 1, w.k, w.B, w.ratio, w.layout, w.seed, oracle_rows=False, policy=policy, policy_seed=7)
    try:
        for t in range(x.shape[0]):
            p.step(0, x[t], check_state=False)
            if t % 8 == 7:
                p.check_state(0, w.n, sample_rows=128)
    finally:
        p.close()


def test_fifo_append_interleaved_matches_oracle():
    n, B, k, ratio = 3, 48, 20, 4
    cap = ratio * B
    say("FIFO append + resolve vs oracle")
    rng = np.random.default_rng(31)
    hs = hsa.HiSparse(k, B, ratio, n, 1, hsa.LAYOUT_BF16, eviction=hsa.EVICT_FIFO)
    try:
        fill_host_pool(hs, 13)
        host = np.stack([np.stack([hs.host_kv(0, r).copy()]) for r in range(n)])
        orc = oracle.OracleCache(n, 1, B, cap, host=np.ascontiguousarray(host), policy=oracle.FIFO)
        nxt = np.array([5, 50, 100])
        for step in range(30):
            pos = nxt.copy().astype(np.int32)
            nxt += 1
            re = rng.random(n) < 0.3                               # rewrite a possibly resident token
            pos[re] = rng.integers(0, cap, size=int(re.sum()))
            rows = rng.integers(0, 256, size=(n, 1152), dtype=np.uint8)
            s_o = orc.append(0, pos, rows)
            s_d = hs.append(0, torch.from_numpy(pos).cuda(), torch.from_numpy(rows).cuda())
            S = np.stack([rng.choice(cap, k, replace=False) for _ in range(n)]).astype(np.int32)
            for r in range(n):
                if pos[r] not in S[r] and rng.random() < 0.7:
                    S[r, 0] = pos[r]
            slots_d, miss_d = hs.resolve(0, torch.from_numpy(S).cuda())
            slots_o, miss_o = orc.resolve(0, S)
            torch.cuda.synchronize()
            assert (s_d.cpu().numpy() == s_o).all()
            assert (slots_d.cpu().numpy() == slots_o).all() and (miss_d.cpu().numpy() == miss_o).all()
            st = hs.state(0)
            assert (st["page_table"].cpu().numpy() == orc.PT[:, 0]).all()
            assert (st["slot_stamp"].cpu().numpy().astype(np.int64) == orc.ST[:, 0]).all()
            rm = st["slot_owner"].cpu().numpy()
            assert (rm == orc.RM[:, 0]).all()
            order = st["lru_order"].cpu().numpy()
            stamp = st["slot_stamp"].cpu().numpy()
            for r in range(n):
                assert (order[r] == np.lexsort((np.arange(B), stamp[r].astype(np.int64)))).all()
            buf = st["kv_buffer"].cpu().numpy()
            for r in range(n):
                occ = np.nonzero(rm[r] >= 0)[0]
                assert (buf[r, occ] == orc.dev[r, 0, occ]).all()
    finally:
        hs.close()


def test_random_policy_rejects_append_and_differs_from_lru():
    n, B, k = 2, 64, 16
    rnd = hsa.HiSparse(k, B, 4, n, 1, hsa.LAYOUT_BF16, eviction=hsa.EVICT_RANDOM, eviction_seed=3)
    lru = hsa.HiSparse(k, B, 4, n, 1, hsa.LAYOUT_BF16)
    try:
        with pytest.raises(hsa.HSError):
            rnd.append(0, torch.zeros(n, dtype=torch.int32, device="cuda"),
                       torch.zeros(n, 1152, dtype=torch.uint8, device="cuda"))
        rng = np.random.default_rng(8)
        differ = False
        for t in range(20):
            S = torch.from_numpy(np.stack([rng.choice(4 * B, k, replace=False) for _ in range(n)])
                                 .astype(np.int32)).cuda()
            a, _ = rnd.resolve(0, S)
            b, _ = lru.resolve(0, S)
            differ |= not torch.equal(a, b)
        assert differ
    finally:
        rnd.close()
        lru.close()
