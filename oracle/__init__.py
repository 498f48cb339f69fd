"""CPU oracle for the HiSparse hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the package's ``smoke()`` check and the benchmark's
``cpu_baseline`` leg may import this package.  The device library never loads
it, and it shares no code with the device library.

``hs_oracle.c`` is the plain C oracle (literal LRU resolve with qsort, fp64
attention); :mod:`oracle.naive` is a second, pure-Python restatement used to pin
it.  This module is the ctypes loader plus a small stateful wrapper,
:class:`OracleCache`, that holds one state per (request, layer) exactly as the
method defines it: page table, slot owner map, recency stamps, step counter and
(optionally) the bytes of the device slots.

Pinned by tests/test_oracle_pins.py (closed forms, brute force over
presentation orders, a textbook LRU for k = 1, torch fp64 attention, the
torch E4M3FN decode table, and the exactness property of the paper abstract).

Page-granular selections (paper abstract: the method is evaluated with the NSA and
Quest families, which select blocks of consecutive tokens): with ``page_tokens`` P > 1
the cached unit is a page of P consecutive tokens -- the page table maps page -> slot,
a slot holds the P rows of its page, a miss fetches the whole page, and the same
replacement rule applies to pages.  Attention then runs over every token of the
resolved pages (:meth:`OracleCache.attend`), or over those before each request's
context length (:meth:`OracleCache.attend_pages`).  Pinned by
tests/test_oracle_page_pins.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from functools import lru_cache

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# HS_ORACLE_LIB points at another build of hs_oracle.c (the sanitizer test's instrumented one)
_SO = os.environ.get("HS_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "hs_oracle.c")

OK, BAD_TOKEN, DUPLICATE, NO_ROOM, NOMEM, BAD_POLICY = 0, -1, -2, -3, -4, -5
LRU, FIFO, RANDOM = 0, 1, 2     # eviction policies (hs_oracle.c)
ENTRY_BYTES = {0: 1152, 1: 656}


class OracleError(ValueError):
    pass


def build(force: bool = True) -> str:
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


@lru_cache(maxsize=1)
def lib():
    if not os.path.exists(_SO):
        build(force=False)
    L = ctypes.CDLL(_SO)
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    L.orc_resolve.restype = ctypes.c_int
    u64 = ctypes.c_uint64
    L.orc_resolve.argtypes = [i64, i64, i64, p, p, p, i64, p, p, p, p, p, i64, ctypes.c_int, u64, i64]
    L.orc_resolve_batch.restype = ctypes.c_int
    L.orc_resolve_batch.argtypes = [i64, i64, i64, i64, p, p, p, p, p, p, p, p, p, i64, ctypes.c_int, ctypes.c_int,
                                    u64, i64, i64]
    L.orc_random_perm.restype = ctypes.c_uint32
    L.orc_random_perm.argtypes = [u64, i64, i64, ctypes.c_uint32, ctypes.c_uint32]
    L.orc_append.restype = ctypes.c_int
    L.orc_append.argtypes = [i64, i64, p, p, p, i64, ctypes.c_int32, p, p, p, i64, p, ctypes.c_int]
    L.orc_e4m3_decode.restype = ctypes.c_double
    L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    L.orc_attend.restype = ctypes.c_int
    L.orc_attend.argtypes = [i64, ctypes.c_int, i64, p, p, p, i64, ctypes.c_double, p, p]
    L.orc_attend_batch.restype = ctypes.c_int
    L.orc_attend_batch.argtypes = [i64, i64, ctypes.c_int, i64, p, p, p, i64, i64, ctypes.c_double, p, p,
                                   ctypes.c_int]
    return L


def _ptr(a):
    return None if a is None else a.ctypes.data


def e4m3_decode(code: int) -> float:
    return lib().orc_e4m3_decode(code)


def random_perm(seed: int, rl: int, t: int, N: int, x: int) -> int:
    """The RANDOM policy's permutation of [0, N) for request-layer rl at step t, at x."""
    return lib().orc_random_perm(seed, rl, t, N, x)


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


class OracleCache:
    """Per-(request, layer) cache states, resolved and attended by the C oracle.

    host: optional [n][L][cap * page_tokens][E] uint8 array holding each request's
    full KV history, one row per token; when given, the oracle also keeps the device-slot
    bytes ``dev[n][L][B][page_tokens * E]`` and fills them on every miss.  policy: LRU
    (the method), or FIFO / RANDOM (seeded) for the eviction-policy study.

    page_tokens P: tokens per cached unit.  With P > 1, selections, B and cap count pages
    (page c = tokens cP .. cP + P - 1) and every table entry is a page.
    """

    def __init__(self, n: int, L: int, B: int, cap: int, layout: int = 0, host: np.ndarray | None = None,
                 threads: int | None = None, policy: int = LRU, seed: int = 0, page_tokens: int = 1):
        if B <= 0 or cap <= 0 or n <= 0 or L <= 0 or page_tokens <= 0:
            raise OracleError("bad shape")
        self.n, self.L, self.B, self.cap, self.layout = n, L, B, cap, layout
        self.P = page_tokens
        self.E_tok = ENTRY_BYTES[layout]
        self.E = self.E_tok * self.P          # bytes of one cached unit: the P rows of a page, in order
        self.PT = np.full((n, L, cap), -1, dtype=np.int32)
        self.RM = np.full((n, L, B), -1, dtype=np.int32)
        self.ST = np.full((n, L, B), -1, dtype=np.int64)
        self.t = np.zeros((n, L), dtype=np.int64)
        self.host = host
        if host is not None:
            assert host.shape == (n, L, cap * self.P, self.E_tok) and host.dtype == np.uint8 and host.flags.c_contiguous
            self.dev = np.zeros((n, L, B, self.E), dtype=np.uint8)
        else:
            self.dev = None
        self.threads = threads or default_threads()
        self.policy, self.seed = policy, seed

    def resolve(self, layer: int, S: np.ndarray, requests: int | None = None):
        """Resolve S[n_req][k] for layer ``layer``; returns (slots[n_req][k] int32, miss[n_req] int64)."""
        S = np.ascontiguousarray(S, dtype=np.int32)
        nr = S.shape[0] if requests is None else requests
        k = S.shape[1]
        slots = np.empty((nr, k), dtype=np.int32)
        miss = np.empty(nr, dtype=np.int64)
        PT = np.ascontiguousarray(self.PT[:nr, layer])
        RM = np.ascontiguousarray(self.RM[:nr, layer])
        ST = np.ascontiguousarray(self.ST[:nr, layer])
        t = np.ascontiguousarray(self.t[:nr, layer])
        dev = host = None
        if self.dev is not None:
            dev = np.ascontiguousarray(self.dev[:nr, layer])
            host = np.ascontiguousarray(self.host[:nr, layer])
        rc = lib().orc_resolve_batch(nr, self.B, self.cap, k, _ptr(PT), _ptr(RM), _ptr(ST), _ptr(t), _ptr(S),
                                     _ptr(slots), _ptr(miss), _ptr(dev), _ptr(host), self.E, self.threads,
                                     self.policy, self.seed, self.L, layer)
        if rc != OK:
            raise OracleError(f"invalid selection (code {rc})")
        self.PT[:nr, layer] = PT
        self.RM[:nr, layer] = RM
        self.ST[:nr, layer] = ST
        if dev is not None:
            self.dev[:nr, layer] = dev
        self.t[:nr, layer] += 1
        return slots, miss

    def append(self, layer: int, pos: np.ndarray, rows: np.ndarray) -> np.ndarray:
        """Write-through append of one new token per request: pos[n_req] (-1 = none), rows[n_req][E].

        Each row goes to the host history (``host``, when kept) and the token becomes
        resident (``orc_append``); returns the slot of each appended token (-1 for none).
        The step counters do not move: the stamp given is the next resolve's step."""
        if self.P != 1:
            return self._append_pages(layer, pos, rows)
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        rows = np.ascontiguousarray(rows, dtype=np.uint8)
        assert rows.shape == (pos.shape[0], self.E)
        out = np.full(pos.shape[0], -1, dtype=np.int32)
        for r in range(pos.shape[0]):
            if pos[r] == -1:
                continue
            PT = np.ascontiguousarray(self.PT[r, layer])
            RM = np.ascontiguousarray(self.RM[r, layer])
            ST = np.ascontiguousarray(self.ST[r, layer])
            dev = None if self.dev is None else np.ascontiguousarray(self.dev[r, layer])
            host = None if self.host is None else np.ascontiguousarray(self.host[r, layer])
            slot = ctypes.c_int32(-1)
            rc = lib().orc_append(self.B, self.cap, _ptr(PT), _ptr(RM), _ptr(ST), int(self.t[r, layer]), int(pos[r]),
                                  _ptr(rows[r]), _ptr(dev), _ptr(host), self.E, ctypes.byref(slot), self.policy)
            if rc != OK:
                raise OracleError(f"invalid append (code {rc})")
            self.PT[r, layer], self.RM[r, layer], self.ST[r, layer] = PT, RM, ST
            if dev is not None:
                self.dev[r, layer] = dev
            if host is not None:
                self.host[r, layer] = host
            out[r] = slot.value
        return out

    def _append_pages(self, layer: int, pos: np.ndarray, rows: np.ndarray) -> np.ndarray:
        """Write-through append with pages: each new token's row goes to its history position,
        and into its page's slot when that page is resident (at row offset pos mod P).  No
        table changes: a page that is not resident is fetched whole, new row included, when a
        selection names it.  Returns the page's slot (-1 when not resident or no token)."""
        pos = np.asarray(pos, dtype=np.int64)
        rows = np.ascontiguousarray(rows, dtype=np.uint8)
        assert rows.shape == (pos.shape[0], self.E_tok)
        out = np.full(pos.shape[0], -1, dtype=np.int32)
        for r in range(pos.shape[0]):
            p = int(pos[r])
            if p == -1:
                continue
            if p < 0 or p >= self.cap * self.P:
                raise OracleError("append position out of range")
            if self.host is not None:
                self.host[r, layer, p] = rows[r]
            c, o = p // self.P, p % self.P
            j = int(self.PT[r, layer, c])
            if j >= 0:
                if self.dev is not None:
                    self.dev[r, layer, j, o * self.E_tok:(o + 1) * self.E_tok] = rows[r]
                out[r] = j
        return out

    def attend(self, layer: int, q: np.ndarray, slots: np.ndarray, scale: float):
        """q[n_req][H][576] bf16 bits (uint16) -> (out[n_req][H][512] f64, lse[n_req][H] f64).

        With pages, every token of every resolved page takes part."""
        if self.P != 1:
            return self.attend_pages(layer, q, slots, None, None, scale)
        if self.dev is None:
            raise OracleError("attention needs the slot bytes (construct with host=...)")
        q = np.ascontiguousarray(q, dtype=np.uint16)
        slots = np.ascontiguousarray(slots, dtype=np.int32)
        nr, H = q.shape[0], q.shape[1]
        dev = np.ascontiguousarray(self.dev[:nr, layer])
        return attend_rows(q, slots, dev, self.layout, scale, self.threads)

    def attend_pages(self, layer: int, q: np.ndarray, slots: np.ndarray, sel: np.ndarray | None,
                     lens: np.ndarray | None, scale: float):
        """Attention over the tokens of the resolved pages: slots[n_req][k] page slots (-1
        skipped); with sel (the page selection) and lens (context length in tokens per
        request), only tokens at positions < lens[r] take part."""
        if self.dev is None:
            raise OracleError("attention needs the slot bytes (construct with host=...)")
        q = np.ascontiguousarray(q, dtype=np.uint16)
        nr = q.shape[0]
        idx = page_token_rows(slots, sel, lens, self.P)
        rows = np.ascontiguousarray(self.dev[:nr, layer]).reshape(nr, self.B * self.P, self.E_tok)
        return attend_rows(q, idx, rows, self.layout, scale, self.threads)


def page_token_rows(slots: np.ndarray, sel: np.ndarray | None, lens: np.ndarray | None, P: int) -> np.ndarray:
    """Token rows of the resolved pages, in selection order: entry i * P + o is row
    slots[r][i] * P + o of the request's slot rows (a slot holds its page's P rows in
    position order), or -1 when the page is padding or, given sel and lens, when its
    position sel[r][i] * P + o is not below lens[r]."""
    slots = np.asarray(slots)
    n, k = slots.shape
    idx = np.full((n, k * P), -1, dtype=np.int32)
    for r in range(n):
        for i in range(k):
            j = int(slots[r, i])
            if j < 0:
                continue
            for o in range(P):
                if sel is not None:
                    c = int(sel[r, i])
                    if c < 0 or c * P + o >= int(lens[r]):
                        continue
                idx[r, i * P + o] = j * P + o
    return idx


def attend_rows(q: np.ndarray, idx: np.ndarray, rows: np.ndarray, layout: int, scale: float,
                threads: int | None = None):
    """Attention of q[n][H][576] over rows[n][R][E] picked by idx[n][k] (-1 skipped), fp64."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    n, H = q.shape[0], q.shape[1]
    k = idx.shape[1]
    E = rows.shape[-1]
    if idx.size and int(idx.max()) >= rows.shape[1]:
        raise OracleError("row index out of range")
    out = np.empty((n, H, 512), dtype=np.float64)
    lse = np.empty((n, H), dtype=np.float64)
    rc = lib().orc_attend_batch(n, k, layout, H, _ptr(q), _ptr(idx), _ptr(rows), rows.shape[1] * E, E, scale,
                                _ptr(out), _ptr(lse), threads or default_threads())
    if rc != OK:
        raise OracleError(f"attention failed (code {rc})")
    return out, lse
