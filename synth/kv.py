"""Seeded synthetic KV rows and decode queries (input generator only).

The rows stand in for the KV entries that a DeepSeek-style MLA layer writes:
576 values per token (512 latent + 64 rope), stored either as 576 bf16
(1152 bytes) or as 512 FP8 E4M3FN latent codes with one fp32 scale per 128
latent values plus 64 bf16 rope values (656 bytes).  Every element is an
inverse-CDF draw of N(0, 1) through a 65536-entry quantile table, indexed by a
counter-based hash of (seed, request, layer, position, element), so any row can
be regenerated on its own.

``synth/kvgen.c`` is the fast, threaded writer used for large host pools;
:func:`row_numpy` is a slow NumPy restatement of the same recipe that the tests
compare it with byte for byte.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from functools import lru_cache

import numpy as np
from scipy.special import ndtri

LAYOUT_BF16 = 0   # 576 x bf16 = 1152 bytes
LAYOUT_FP8 = 1    # 512 x e4m3 + 4 x fp32 + 64 x bf16 = 656 bytes
ENTRY_BYTES = {LAYOUT_BF16: 1152, LAYOUT_FP8: 656}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_SRC = os.path.join(_HERE, "kvgen.c")

M64 = (1 << 64) - 1
QUERY_TAG = 0x51E7C0DE


def build(force: bool = True) -> str:
    """Compile the threaded row writer with gcc (host code only)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


@lru_cache(maxsize=1)
def _lib():
    if not os.path.exists(_SO):
        build(force=False)
    lib = ctypes.CDLL(_SO)
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    for name in ("synth_fill_rows", "synth_rows_at"):
        fn = getattr(lib, name)
        fn.restype = None
    lib.synth_fill_rows.argtypes = [ctypes.c_uint64, i64, i64, i64, i64, ctypes.c_int, p, p, p, i64, ctypes.c_int]
    lib.synth_rows_at.argtypes = [ctypes.c_uint64, i64, i64, p, i64, ctypes.c_int, p, p, p, i64, ctypes.c_int]
    lib.synth_fill_rows_split.restype = None
    lib.synth_fill_rows_split.argtypes = [ctypes.c_uint64, i64, i64, i64, i64, ctypes.c_int, p, p, p, i64, i64, p,
                                          i64, ctypes.c_int]
    lib.synth_e4m3_encode.restype = ctypes.c_uint8
    lib.synth_e4m3_encode.argtypes = [ctypes.c_float]
    lib.synth_mix64.restype = ctypes.c_uint64
    lib.synth_mix64.argtypes = [ctypes.c_uint64]
    return lib


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@lru_cache(maxsize=1)
def normal_tables():
    """65536 equiprobable standard-normal quantiles, as fp32 and as bf16 bits."""
    q = ndtri((np.arange(65536, dtype=np.float64) + 0.5) / 65536.0).astype(np.float32)
    return np.ascontiguousarray(f32_to_bf16_bits(q)), np.ascontiguousarray(q)


def fill_rows(seed: int, r: int, l: int, pos0: int, count: int, layout: int, dst_ptr: int, stride: int,
              nthreads: int | None = None) -> None:
    """Write rows pos0..pos0+count-1 at ``dst_ptr + i*stride`` (any host memory)."""
    tb, tf = normal_tables()
    nt = nthreads or min(16, os.cpu_count() or 1)
    _lib().synth_fill_rows(seed, r, l, pos0, count, layout, tb.ctypes.data, tf.ctypes.data,
                           ctypes.c_void_p(dst_ptr), stride, nt)


def fill_rows_split(seed: int, r: int, l: int, pos0: int, count: int, layout: int, dst_ptr: int, stride: int,
                    body: int, tail_ptr: int, tail_stride: int, nthreads: int | None = None) -> None:
    """The rows of :func:`fill_rows`, split: the first ``body`` bytes of row i at
    ``dst_ptr + i*stride``, the remaining bytes at ``tail_ptr + i*tail_stride``."""
    if not 0 < body < ENTRY_BYTES[layout]:
        raise ValueError("body must lie strictly inside a row")
    tb, tf = normal_tables()
    nt = nthreads or min(16, os.cpu_count() or 1)
    _lib().synth_fill_rows_split(seed, r, l, pos0, count, layout, tb.ctypes.data, tf.ctypes.data,
                                 ctypes.c_void_p(dst_ptr), stride, body, ctypes.c_void_p(tail_ptr), tail_stride, nt)


def rows_at(seed: int, r: int, l: int, positions, layout: int, nthreads: int | None = None) -> np.ndarray:
    """Rows for explicit positions, as a [len, entry_bytes] uint8 array."""
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int64).reshape(-1))
    E = ENTRY_BYTES[layout]
    out = np.empty((pos.size, E), dtype=np.uint8)
    if pos.size:
        tb, tf = normal_tables()
        nt = nthreads or min(16, os.cpu_count() or 1)
        _lib().synth_rows_at(seed, r, l, pos.ctypes.data, pos.size, layout, tb.ctypes.data, tf.ctypes.data,
                             out.ctypes.data, E, nt)
    return out


def pool(seed: int, r: int, l: int, cap: int, layout: int) -> np.ndarray:
    """A whole [cap, entry_bytes] history for one (request, layer) as a NumPy array."""
    E = ENTRY_BYTES[layout]
    out = np.empty((cap, E), dtype=np.uint8)
    fill_rows(seed, r, l, 0, cap, layout, out.ctypes.data, E)
    return out


# ---- slow NumPy restatement of kvgen.c, used only to check it -------------------------------

def mix64_np(z):
    z = (np.asarray(z, dtype=np.uint64) + np.uint64(0x9E3779B97F4A7C15))
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def _idx16(key, nelem: int) -> np.ndarray:
    e = np.arange(nelem, dtype=np.uint64)
    u = mix64_np(np.uint64(key) + (e >> np.uint64(2)))
    return ((u >> (np.uint64(16) * (e & np.uint64(3)))) & np.uint64(0xFFFF)).astype(np.int64)


def row_key_np(seed: int, r: int, l: int, pos: int) -> np.uint64:
    with np.errstate(over="ignore"):
        k = mix64_np(np.uint64(seed))
        k = mix64_np(k ^ np.uint64(r))
        k = mix64_np(k ^ np.uint64(l))
        return mix64_np(k ^ np.uint64(pos))


def e4m3_encode_np(v: np.ndarray) -> np.ndarray:
    """RNE, saturating fp32 -> E4M3FN codes (finite inputs)."""
    v = np.asarray(v, dtype=np.float32)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
    a = np.abs(v)
    _, e2 = np.frexp(a)
    E = np.maximum(e2.astype(np.int64) - 1, -6)
    q = np.rint(np.ldexp(a, (3 - E).astype(np.int32))).astype(np.float32)
    sub = (E == -6) & (q < 8)
    bump = (~sub) & (q >= 16)
    q = np.where(bump, 8, q)
    E = np.where(bump, E + 1, E)
    code = np.where(sub, q.astype(np.int64), ((E + 7) << 3) | (q.astype(np.int64) - 8))
    code = np.where(a >= 448.0, 0x7E, np.minimum(code, 0x7E))
    code = np.where(a == 0, 0, code)
    return (sign | code).astype(np.uint8)


def row_numpy(seed: int, r: int, l: int, pos: int, layout: int) -> np.ndarray:
    tb, tf = normal_tables()
    with np.errstate(over="ignore"):
        key = row_key_np(seed, r, l, pos)
        idx = _idx16(key, 576)
    if layout == LAYOUT_BF16:
        return tb[idx].view(np.uint8).copy()
    x = tf[idx[:512]].reshape(4, 128)
    amax = np.max(np.abs(x), axis=1)
    s = (amax / np.float32(448.0)).astype(np.float32)
    codes = e4m3_encode_np((x / s[:, None]).astype(np.float32)).reshape(-1)
    rope = tb[idx[512:]]
    return np.concatenate([codes, s.view(np.uint8), rope.view(np.uint8)])


# ---- decode queries ------------------------------------------------------------------------

def queries(seed: int, step: int, n: int, layer: int, heads: int, dim: int = 576) -> np.ndarray:
    """q[n][heads][dim] as bf16 bit patterns (uint16): N(0,1) through the quantile table."""
    tb, _ = normal_tables()
    out = np.empty((n, heads, dim), dtype=np.uint16)
    with np.errstate(over="ignore"):
        base = mix64_np(np.uint64(seed) ^ np.uint64(QUERY_TAG))
        base = mix64_np(base ^ np.uint64(step))
        base = mix64_np(base ^ np.uint64(layer))
        e = np.arange(heads * dim, dtype=np.uint64)
        for r in range(n):
            key = mix64_np(base ^ np.uint64(r))
            u = mix64_np(key + (e >> np.uint64(2)))
            idx = ((u >> (np.uint64(16) * (e & np.uint64(3)))) & np.uint64(0xFFFF)).astype(np.int64)
            out[r] = tb[idx].reshape(heads, dim)
    return out
