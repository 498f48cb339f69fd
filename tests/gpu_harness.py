"""Shared helpers of the GPU parity tests: set up a handle and an oracle on the same
seeded inputs, step both, and compare.  Inputs come only from ``synth``; expected
values come only from ``oracle``."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import hierarchical_kv_cache_hs_amd as hsa
import oracle
from synth import kv as skv
from synth import trace as tr


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def fill_host_pool(hs: hsa.HiSparse, seed: int, requests: int | None = None, layers: int | None = None):
    """Writes every history row of the handle from the seeded generator; with the resident-tail
    layout the host part of each row goes to the host pool and the rest to the tail plane."""
    for l in range(hs.L if layers is None else layers):
        tails = hs.tail_plane(l) if hs.tail_bytes else None
        for r in range(hs.n if requests is None else requests):
            ptr, cap, stride = hs.host_kv_ptr(l, r)
            if tails is None:
                skv.fill_rows(seed, r, l, 0, cap, hs.layout, ptr, stride)
            else:
                stage = np.empty((cap, hs.tail_bytes), dtype=np.uint8)
                skv.fill_rows_split(seed, r, l, 0, cap, hs.layout, ptr, stride, stride, stage.ctypes.data,
                                    hs.tail_bytes)
                tails[r].copy_(torch.from_numpy(stage))
    torch.cuda.synchronize()


def history(hs: hsa.HiSparse, layer: int, request: int) -> np.ndarray:
    """[capacity][entry bytes] copy of a request's whole history rows: the host pool, joined
    with the tail plane under the resident-tail layout."""
    host = hs.host_kv(layer, request).copy()
    if not hs.tail_bytes:
        return host
    return np.concatenate([host, hs.tail_plane(layer)[request].cpu().numpy()], axis=1)


def oracle_host(seed: int, n: int, L: int, cap: int, layout: int) -> np.ndarray:
    E = skv.ENTRY_BYTES[layout]
    host = np.empty((n, L, cap, E), dtype=np.uint8)
    for r in range(n):
        for l in range(L):
            skv.fill_rows(seed, r, l, 0, cap, layout, host[r, l].ctypes.data, E)
    return host


def lru_order_ok(stamp: np.ndarray, order: np.ndarray) -> bool:
    """order must be the slots sorted by (stamp, slot) -- a property of the device design aid."""
    B = stamp.shape[-1]
    for r in range(stamp.shape[0]):
        expect = np.lexsort((np.arange(B), stamp[r].astype(np.int64)))
        if not (order[r] == expect).all():
            return False
    return True


class Pair:
    """A device handle and the oracle, fed the same trace."""

    def __init__(self, n, L, k, B, ratio, layout, seed, heads=0, flags=0, oracle_rows=True, requests=None,
                 split=False, policy=0, policy_seed=0, page_tokens=1):
        self.split, self.policy, self.P = split, policy, page_tokens
        self.hs = hsa.HiSparse(top_k=k, device_buffer_size=B, host_to_device_ratio=ratio, max_requests=n,
                               num_layers=L, layout=layout, num_heads=heads, flags=flags, eviction=policy,
                               eviction_seed=policy_seed, page_tokens=page_tokens)
        self.seed, self.n, self.L, self.k, self.B, self.layout = seed, n, L, k, B, layout
        self.cap = ratio * B
        fill_host_pool(self.hs, seed)
        host = oracle_host(seed, n, L, self.cap * page_tokens, layout) if oracle_rows else None
        self.orc = oracle.OracleCache(n, L, B, self.cap, layout=layout, host=host, policy=policy, seed=policy_seed,
                                      page_tokens=page_tokens)
        self.E = skv.ENTRY_BYTES[layout] * page_tokens     # bytes of a slot: the P rows of a page

    def step(self, layer: int, S: np.ndarray, check_state: bool):
        sel = torch.from_numpy(np.ascontiguousarray(S, dtype=np.int32)).cuda()
        slots_d, miss_d = self.hs.resolve(layer, sel, split=self.split)
        slots_o, miss_o = self.orc.resolve(layer, S)
        torch.cuda.synchronize()
        slots_g = slots_d.cpu().numpy()
        miss_g = miss_d.cpu().numpy()
        assert (slots_g == slots_o).all(), f"slots differ at layer {layer}"
        assert (miss_g == miss_o).all(), f"miss counts differ at layer {layer}"
        if check_state:
            self.check_state(layer, S.shape[0])
        return slots_g, miss_g

    def check_state(self, layer: int, nr: int, rows: bool = True, sample_rows: int | None = None):
        st = self.hs.state(layer)
        pt = st["page_table"][:nr].cpu().numpy()
        rm = st["slot_owner"][:nr].cpu().numpy()
        stamp = st["slot_stamp"][:nr].cpu().numpy()
        order = st["lru_order"][:nr].cpu().numpy()
        assert (pt == self.orc.PT[:nr, layer]).all(), "page table differs"
        assert (rm == self.orc.RM[:nr, layer]).all(), "slot owners differ"
        assert (stamp.astype(np.int64) == self.orc.ST[:nr, layer]).all(), "stamps differ"
        assert (st["step"][:nr].cpu().numpy() == self.orc.t[:nr, layer]).all(), "step counters differ"
        if self.policy != hsa.EVICT_RANDOM:     # RANDOM keeps no order array
            assert lru_order_ok(stamp, order), "LRU order is not (stamp, slot) sorted"
        if rows:
            buf = st["kv_buffer"][:nr, :, : self.E].cpu().numpy()
            for r in range(nr):
                occ = np.nonzero(rm[r] >= 0)[0]
                if sample_rows is not None and occ.size > sample_rows:
                    occ = np.random.default_rng(r).choice(occ, sample_rows, replace=False)
                if self.orc.dev is not None:
                    assert (buf[r, occ] == self.orc.dev[r, layer, occ]).all(), f"slot bytes differ (request {r})"
                else:
                    P = self.P
                    tokens = (rm[r, occ][:, None].astype(np.int64) * P + np.arange(P)).reshape(-1)
                    expect = skv.rows_at(self.seed, r, layer, tokens, self.layout).reshape(occ.size, self.E)
                    assert (buf[r, occ] == expect).all(), f"slot bytes differ (request {r})"

    def close(self):
        self.hs.close()


def trace_for(workload, steps=None, requests=None):
    t0 = time.time()
    x = tr.generate(workload.trace_spec(), steps=steps, requests=requests)
    say(f"trace {workload.name}: {x.shape} in {time.time() - t0:.1f}s")
    return x
