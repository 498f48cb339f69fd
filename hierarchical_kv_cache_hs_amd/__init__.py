"""MI355X-native HiSparse hot path: Python binding of libhs.so (include/hs.h).

Argument marshalling only.  Every step of the path -- hit detection, LRU
replacement, page-table update, host-to-device fetch, sparse MLA attention --
runs in the library's HIP kernels.  PyTorch supplies device memory (the
library's device block is a torch allocation) and streams.  There is no CPU
fallback: if libhs.so is missing the import fails.

    hs = HiSparse(top_k=2048, device_buffer_size=4096, host_to_device_ratio=8,
                  max_requests=64, num_layers=1, layout=LAYOUT_BF16)
    hs.host_kv(layer, request)[:] = rows           # pinned host history
    slots, miss = hs.resolve(layer, sel)           # sel: int32 cuda [n_req][top_k]
    out, lse = hs.attend(layer, q, slots, scale)   # q: bf16 cuda [n_req][H][576]

With page_tokens=P > 1 the cached unit is a page of P consecutive tokens: selections,
top_k, the buffer size and the capacity count pages; the host history stays one row
per token, and attend / attend_pages read every token of the resolved pages.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhs.so")

LAYOUT_BF16 = 0      # HS_KV_BF16_576
LAYOUT_FP8 = 1       # HS_KV_FP8_MLA_656
ENTRY_BYTES = {LAYOUT_BF16: 1152, LAYOUT_FP8: 656}
FLAG_NO_IO = 0x1
FLAG_ATTN_OUT_F32 = 0x2   # attention output in fp32 (P carried in fp32)
FLAG_RESIDENT_TAIL = 0x4  # 656-byte rows: host keeps 640 bytes per row, the last 16 stay on the device
EVICT_LRU, EVICT_FIFO, EVICT_RANDOM = 0, 1, 2   # hs_eviction
DEVERR_TOKEN_RANGE = 0x1
DEVERR_DUPLICATE = 0x2

HS_OK, HS_ERR_INVALID_ARG, HS_ERR_OUT_OF_MEMORY, HS_ERR_UNSUPPORTED, HS_ERR_HIP, HS_ERR_DEVICE = range(6)

SYMBOLS = ("hs_create", "hs_resolve", "hs_resolve_tables", "hs_fetch_misses", "hs_attend", "hs_attend_pages",
           "hs_destroy",
           "hs_append", "hs_offload", "hs_topk",
           "hs_device_bytes", "hs_host_bytes", "hs_host_kv",
           "hs_device_state", "hs_reset_requests", "hs_get_device_error", "hs_status_string",
           "hs_last_error_message", "hs_stream_read", "hs_attend_resident", "hs_attend_fetched",
           "hs_attend_noalloc", "hs_topk_hinted")


class Config(ctypes.Structure):
    _fields_ = [("top_k", ctypes.c_int32), ("device_buffer_size", ctypes.c_int32),
                ("host_to_device_ratio", ctypes.c_int32), ("max_requests", ctypes.c_int32),
                ("num_layers", ctypes.c_int32), ("layout", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("device_mem", ctypes.c_void_p), ("device_mem_bytes", ctypes.c_size_t),
                ("eviction", ctypes.c_int32), ("eviction_seed", ctypes.c_uint64), ("page_tokens", ctypes.c_int32)]


class StateView(ctypes.Structure):
    _fields_ = [("page_table", ctypes.c_void_p), ("slot_owner", ctypes.c_void_p), ("slot_stamp", ctypes.c_void_p),
                ("lru_order", ctypes.c_void_p), ("step", ctypes.c_void_p), ("kv_buffer", ctypes.c_void_p),
                ("capacity", ctypes.c_int64), ("slot_stride", ctypes.c_int64), ("entry_bytes", ctypes.c_int64),
                ("request_stride", ctypes.c_int64), ("page_tokens", ctypes.c_int64),
                ("fresh_slots", ctypes.c_void_p), ("tail_plane", ctypes.c_void_p), ("tail_bytes", ctypes.c_int64)]


class HSError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


_lib_cache = None


def lib():
    """The loaded libhs.so; raises if it has not been built (no fallback)."""
    global _lib_cache
    if _lib_cache is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m hierarchical_kv_cache_hs_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        p, i32 = ctypes.c_void_p, ctypes.c_int32
        L.hs_device_bytes.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(ctypes.c_size_t)]
        L.hs_host_bytes.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(ctypes.c_size_t)]
        L.hs_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(p)]
        L.hs_resolve.argtypes = [p, i32, i32, p, p, p, p]
        L.hs_resolve_tables.argtypes = [p, i32, i32, p, p, p, p]
        L.hs_fetch_misses.argtypes = [p, i32, i32, p]
        L.hs_append.argtypes = [p, i32, i32, p, p, ctypes.c_int64, p, p]
        L.hs_topk.argtypes = [p, i32, p, ctypes.c_int64, p, p, p]
        L.hs_topk_hinted.argtypes = [p, i32, p, ctypes.c_int64, p, p, p, p]
        L.hs_offload.argtypes = [p, i32, i32, ctypes.c_int64, ctypes.c_int64, p, ctypes.c_int64, p]
        L.hs_attend.argtypes = [p, i32, i32, p, p, ctypes.c_float, p, p, p]
        L.hs_attend_pages.argtypes = [p, i32, i32, p, p, p, p, ctypes.c_float, p, p, p]
        L.hs_destroy.argtypes = [p]
        L.hs_stream_read.argtypes = [p, ctypes.c_size_t, p, p]
        L.hs_attend_resident.argtypes = [p, i32, i32, p, p, p, p, ctypes.c_float, p]
        L.hs_attend_fetched.argtypes = [p, i32, i32, p, p, ctypes.c_float, p, p, p]
        L.hs_attend_noalloc.argtypes = [p, i32, i32, i32, p, p, ctypes.c_float, p, p, p]
        L.hs_host_kv.argtypes = [p, i32, i32, ctypes.POINTER(p), ctypes.POINTER(ctypes.c_int64),
                                 ctypes.POINTER(ctypes.c_int64)]
        L.hs_device_state.argtypes = [p, i32, ctypes.POINTER(StateView)]
        L.hs_reset_requests.argtypes = [p, i32, i32, p]
        L.hs_get_device_error.argtypes = [p, ctypes.POINTER(ctypes.c_int32)]
        L.hs_status_string.argtypes = [ctypes.c_int]
        L.hs_status_string.restype = ctypes.c_char_p
        L.hs_last_error_message.argtypes = []
        L.hs_last_error_message.restype = ctypes.c_char_p
        for name in ("hs_device_bytes", "hs_host_bytes", "hs_create", "hs_resolve", "hs_resolve_tables",
                     "hs_fetch_misses", "hs_attend", "hs_attend_pages", "hs_destroy",
                     "hs_host_kv", "hs_device_state", "hs_reset_requests", "hs_get_device_error",
                     "hs_stream_read", "hs_attend_resident", "hs_attend_fetched", "hs_attend_noalloc"):
            getattr(L, name).restype = ctypes.c_int
        _lib_cache = L
    return _lib_cache


def _check(status: int):
    if status != HS_OK:
        raise HSError(status, lib().hs_last_error_message().decode())


def _require(ok: bool, msg: str = "tensor argument of the wrong dtype, shape, layout or size"):
    """Argument check of the binding: the kernels index these tensors with the handle's sizes,
    so a mismatch must stop the call before anything is enqueued (a plain raise, not an
    assert, so it also holds under python -O)."""
    if not ok:
        raise ValueError(msg)


def make_config(top_k, device_buffer_size, host_to_device_ratio, max_requests, num_layers=1, layout=LAYOUT_BF16,
                num_heads=0, flags=0, eviction=0, eviction_seed=0, page_tokens=1) -> Config:
    return Config(top_k, device_buffer_size, host_to_device_ratio, max_requests, num_layers, layout, num_heads,
                  flags, None, 0, eviction, eviction_seed, page_tokens)


def device_bytes(cfg: Config) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().hs_device_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def host_bytes(cfg: Config) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().hs_host_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None):
    """Enqueue the library's dense streaming read of `src` (a measurement helper, not a step
    of the method); `sink` is a one-element int32 cuda tensor the kernel may overwrite."""
    _require(src.is_cuda and src.is_contiguous() and sink.is_cuda and sink.dtype == torch.int32)
    _check(lib().hs_stream_read(src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(),
                                _stream_ptr(stream)))


def _stream_ptr(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


class HiSparse:
    """One handle: per-(request, layer) page tables, LRU state, device slots and pinned host history."""

    def __init__(self, top_k: int, device_buffer_size: int, host_to_device_ratio: int, max_requests: int,
                 num_layers: int = 1, layout: int = LAYOUT_BF16, num_heads: int = 0, flags: int = 0,
                 device: str | torch.device = "cuda", eviction: int = 0, eviction_seed: int = 0,
                 page_tokens: int = 1):
        self.cfg = make_config(top_k, device_buffer_size, host_to_device_ratio, max_requests, num_layers, layout,
                               num_heads, flags, eviction, eviction_seed, page_tokens)
        nbytes = device_bytes(self.cfg)
        self.device = torch.device(device)
        # torch owns the device block; the library lays its tables out inside it
        self.block = torch.zeros(nbytes, dtype=torch.uint8, device=self.device)
        torch.cuda.synchronize(self.device)  # the fill must land before the library initialises its tables
        self.cfg.device_mem = self.block.data_ptr()
        self.cfg.device_mem_bytes = nbytes
        h = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            _check(lib().hs_create(ctypes.byref(self.cfg), ctypes.byref(h)))
        self._h = h
        self.top_k, self.B, self.n, self.L = top_k, device_buffer_size, max_requests, num_layers
        self.layout, self.heads = layout, num_heads
        self.out_dtype = torch.float32 if flags & FLAG_ATTN_OUT_F32 else torch.bfloat16
        self.entry_bytes = ENTRY_BYTES[layout]
        self.tail_bytes = 16 if flags & FLAG_RESIDENT_TAIL else 0   # row bytes kept in the device tail plane
        self.capacity = host_to_device_ratio * device_buffer_size     # page-table entries
        self.page_tokens = page_tokens

    # -- lifetime ------------------------------------------------------------------------------
    def close(self):
        if self._h is not None and self._h.value:
            _check(lib().hs_destroy(self._h))
        self._h = None
        self.block = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    @property
    def handle(self) -> int:
        return self._h.value

    # -- host pool -----------------------------------------------------------------------------
    def host_kv(self, layer: int, request: int) -> np.ndarray:
        """[capacity * page_tokens][entry_bytes] uint8 view of the pinned host rows (one per token);
        with FLAG_RESIDENT_TAIL [capacity][entry_bytes - 16], the rest being in :meth:`tail_plane`."""
        ptr = ctypes.c_void_p()
        cap = ctypes.c_int64()
        stride = ctypes.c_int64()
        _check(lib().hs_host_kv(self._h, layer, request, ctypes.byref(ptr), ctypes.byref(cap), ctypes.byref(stride)))
        buf = (ctypes.c_uint8 * (cap.value * stride.value)).from_address(ptr.value)
        return np.frombuffer(buf, dtype=np.uint8).reshape(cap.value, stride.value)[:, : self.entry_bytes]

    def tail_plane(self, layer: int) -> torch.Tensor | None:
        """FLAG_RESIDENT_TAIL: [max_requests][capacity][16] uint8 device view of the last 16 bytes
        of every history row of the layer (None without the flag)."""
        return self.state(layer)["tail_plane"]

    def host_kv_ptr(self, layer: int, request: int) -> tuple[int, int, int]:
        ptr = ctypes.c_void_p()
        cap = ctypes.c_int64()
        stride = ctypes.c_int64()
        _check(lib().hs_host_kv(self._h, layer, request, ctypes.byref(ptr), ctypes.byref(cap), ctypes.byref(stride)))
        return ptr.value, cap.value, stride.value

    # -- hot path ------------------------------------------------------------------------------
    def resolve(self, layer: int, sel: torch.Tensor, slots: torch.Tensor | None = None,
                miss: torch.Tensor | None = None, stream=None, split: bool = False):
        """hs_resolve; with split=True, hs_resolve_tables followed by hs_fetch_misses on the same stream."""
        n_req = sel.shape[0]
        _require(sel.dtype == torch.int32 and sel.is_contiguous() and sel.shape[1] == self.top_k)
        if slots is None:
            slots = torch.empty_like(sel)
        if miss is None:
            miss = torch.empty(n_req, dtype=torch.int32, device=sel.device)
        _require(slots.shape == sel.shape and slots.dtype == torch.int32 and slots.is_contiguous())
        _require(miss.dtype == torch.int32 and miss.is_contiguous() and miss.numel() >= n_req)
        self._on_device(sel, slots, miss)
        if split:
            self.resolve_tables(layer, sel, slots, miss, stream)
            self.fetch_misses(layer, n_req, stream)
        else:
            _check(lib().hs_resolve(self._h, layer, n_req, sel.data_ptr(), slots.data_ptr(), miss.data_ptr(),
                                    _stream_ptr(stream)))
        return slots, miss

    def resolve_tables(self, layer: int, sel: torch.Tensor, slots: torch.Tensor, miss: torch.Tensor, stream=None):
        _require(sel.dtype == torch.int32 and sel.is_contiguous() and sel.shape[1] == self.top_k)
        _require(slots.shape == sel.shape and slots.dtype == torch.int32 and slots.is_contiguous())
        _require(miss.dtype == torch.int32 and miss.is_contiguous() and miss.numel() >= sel.shape[0])
        self._on_device(sel, slots, miss)
        _check(lib().hs_resolve_tables(self._h, layer, sel.shape[0], sel.data_ptr(), slots.data_ptr(),
                                       miss.data_ptr(), _stream_ptr(stream)))

    def fetch_misses(self, layer: int, n_req: int, stream=None):
        _check(lib().hs_fetch_misses(self._h, layer, n_req, _stream_ptr(stream)))

    def append(self, layer: int, pos: torch.Tensor, rows: torch.Tensor, slot_out: torch.Tensor | None = None,
               stream=None):
        """hs_append: pos int32 [n_req] (-1 = none), rows uint8 [n_req][>= entry bytes] on the device."""
        n_req = pos.shape[0]
        _require(pos.dtype == torch.int32 and pos.is_contiguous())
        _require(rows.dtype == torch.uint8 and rows.dim() == 2 and rows.shape[0] == n_req and rows.stride(1) == 1)
        if slot_out is None:
            slot_out = torch.empty(n_req, dtype=torch.int32, device=pos.device)
        _require(slot_out.dtype == torch.int32 and slot_out.is_contiguous() and slot_out.numel() >= n_req)
        self._on_device(pos, rows, slot_out)
        _check(lib().hs_append(self._h, layer, n_req, pos.data_ptr(), rows.data_ptr(), rows.stride(0),
                               slot_out.data_ptr(), _stream_ptr(stream)))
        return slot_out

    def topk(self, scores: torch.Tensor, lens: torch.Tensor, sel: torch.Tensor | None = None, stream=None,
             hint: torch.Tensor | None = None):
        """hs_topk: scores float32 [n_req][stride] (stride % 4 == 0), lens int32 [n_req] -> sel [n_req][top_k].
        With ``hint`` (int32 [n_req], in/out, -1 = no guess; keep one per layer across steps),
        hs_topk_hinted: the same selection, in one pass over a row whose guess is right."""
        n_req = scores.shape[0]
        _require(scores.dtype == torch.float32 and scores.dim() == 2 and scores.stride(1) == 1)
        _require(lens.dtype == torch.int32 and lens.is_contiguous() and lens.shape[0] == n_req)
        if sel is None:
            sel = torch.empty(n_req, self.top_k, dtype=torch.int32, device=scores.device)
        _require(sel.shape == (n_req, self.top_k) and sel.dtype == torch.int32 and sel.is_contiguous())
        self._on_device(scores, lens, sel, hint)
        if hint is None:
            _check(lib().hs_topk(self._h, n_req, scores.data_ptr(), scores.stride(0), lens.data_ptr(), sel.data_ptr(),
                                 _stream_ptr(stream)))
        else:
            _require(hint.dtype == torch.int32 and hint.is_contiguous() and hint.shape == (n_req,))
            _check(lib().hs_topk_hinted(self._h, n_req, scores.data_ptr(), scores.stride(0), lens.data_ptr(),
                                        sel.data_ptr(), hint.data_ptr(), _stream_ptr(stream)))
        return sel

    def offload(self, layer: int, request: int, first: int, rows: torch.Tensor, stream=None):
        """hs_offload: rows uint8 [count][>= entry bytes] on the device -> history positions first.."""
        _require(rows.dtype == torch.uint8 and rows.dim() == 2 and rows.stride(1) == 1)
        _check(lib().hs_offload(self._h, layer, request, first, rows.shape[0], rows.data_ptr(), rows.stride(0),
                                _stream_ptr(stream)))

    # -- argument checks shared by the attention calls --------------------------------------------
    def _on_device(self, *ts):
        for t in ts:
            if t is not None:
                _require(t.is_cuda and t.device == self.block.device,
                         f"tensor on {t.device}, handle on {self.block.device}")

    def _attn_io(self, q: torch.Tensor, out, lse):
        """Checks q against the handle's head count and sizes out / lse (the kernels index all
        three with num_heads)."""
        n_req = q.shape[0]
        _require(q.dtype == torch.bfloat16 and q.is_contiguous() and q.dim() == 3 and q.shape[2] == 576)
        # a handle without heads: the library itself refuses (HS_ERR_UNSUPPORTED)
        heads = self.heads if self.heads > 0 else q.shape[1]
        _require(q.shape[1] == heads, f"q has {q.shape[1]} heads, the handle {self.heads}")
        if out is None:
            out = torch.empty(n_req, heads, 512, dtype=self.out_dtype, device=q.device)
        _require(out.dtype == self.out_dtype and out.is_contiguous() and out.shape == (n_req, heads, 512))
        if lse is None:
            lse = torch.empty(n_req, heads, dtype=torch.float32, device=q.device)
        _require(lse.dtype == torch.float32 and lse.is_contiguous() and lse.shape == (n_req, heads))
        self._on_device(q, out, lse)
        return out, lse

    def attend(self, layer: int, q: torch.Tensor, slots: torch.Tensor, scale: float,
               out: torch.Tensor | None = None, lse: torch.Tensor | None = None, stream=None):
        n_req = q.shape[0]
        _require(slots.dtype == torch.int32 and slots.is_contiguous() and slots.shape == (n_req, self.top_k))
        out, lse = self._attn_io(q, out, lse)
        self._on_device(slots)
        _check(lib().hs_attend(self._h, layer, n_req, q.data_ptr(), slots.data_ptr(), float(scale), out.data_ptr(),
                               lse.data_ptr(), _stream_ptr(stream)))
        return out, lse

    def attend_noalloc(self, layer: int, q: torch.Tensor, slots: torch.Tensor, scale: float,
                       out: torch.Tensor | None = None, lse: torch.Tensor | None = None, stream=None):
        """hs_attend_noalloc: hs_attend with q's head count (1..16, any handle) and the split
        partials in the library's static device array; out / lse are allocated here only when
        not given."""
        n_req, heads = q.shape[0], q.shape[1]
        _require(q.dtype == torch.bfloat16 and q.is_contiguous() and q.dim() == 3 and q.shape[2] == 576)
        _require(1 <= heads <= 16)
        _require(slots.dtype == torch.int32 and slots.is_contiguous() and slots.shape == (n_req, self.top_k))
        if out is None:
            out = torch.empty(n_req, heads, 512, dtype=self.out_dtype, device=q.device)
        _require(out.dtype == self.out_dtype and out.is_contiguous() and out.shape == (n_req, heads, 512))
        if lse is None:
            lse = torch.empty(n_req, heads, dtype=torch.float32, device=q.device)
        _require(lse.dtype == torch.float32 and lse.is_contiguous() and lse.shape == (n_req, heads))
        self._on_device(q, slots, out, lse)
        _check(lib().hs_attend_noalloc(self._h, layer, n_req, heads, q.data_ptr(), slots.data_ptr(), float(scale),
                                       out.data_ptr(), lse.data_ptr(), _stream_ptr(stream)))
        return out, lse

    def attend_pages(self, layer: int, q: torch.Tensor, slots: torch.Tensor, sel: torch.Tensor,
                     lens: torch.Tensor, scale: float, out: torch.Tensor | None = None,
                     lse: torch.Tensor | None = None, stream=None):
        """hs_attend_pages: attend cut at lens[r] tokens (sel: the selection slots came from)."""
        n_req = q.shape[0]
        _require(slots.dtype == torch.int32 and slots.is_contiguous() and slots.shape == (n_req, self.top_k))
        _require(sel.dtype == torch.int32 and sel.is_contiguous() and sel.shape == (n_req, self.top_k))
        _require(lens.dtype == torch.int32 and lens.is_contiguous() and lens.dim() == 1 and lens.shape[0] >= n_req)
        out, lse = self._attn_io(q, out, lse)
        self._on_device(slots, sel, lens)
        _check(lib().hs_attend_pages(self._h, layer, n_req, q.data_ptr(), slots.data_ptr(), sel.data_ptr(),
                                     lens.data_ptr(), float(scale), out.data_ptr(), lse.data_ptr(),
                                     _stream_ptr(stream)))
        return out, lse

    def attend_resident(self, layer: int, q: torch.Tensor, slots: torch.Tensor, scale: float,
                        sel: torch.Tensor | None = None, lens: torch.Tensor | None = None, stream=None):
        """hs_attend_resident: after resolve_tables, attend the entries outside this step's victim
        slots into the handle's partials (may run beside fetch_misses of the same layer)."""
        n_req = q.shape[0]
        _require(q.dtype == torch.bfloat16 and q.is_contiguous() and q.dim() == 3 and q.shape[2] == 576)
        _require(self.heads == 0 or q.shape[1] == self.heads, f"q has {q.shape[1]} heads, the handle {self.heads}")
        _require(slots.dtype == torch.int32 and slots.is_contiguous() and slots.shape == (n_req, self.top_k))
        _require((sel is None) == (lens is None))
        if sel is not None:
            _require(sel.dtype == torch.int32 and sel.is_contiguous() and sel.shape == (n_req, self.top_k))
            _require(lens.dtype == torch.int32 and lens.is_contiguous() and lens.dim() == 1 and lens.shape[0] >= n_req)
        self._on_device(q, slots, sel, lens)
        _check(lib().hs_attend_resident(self._h, layer, n_req, q.data_ptr(), slots.data_ptr(),
                                        None if sel is None else sel.data_ptr(),
                                        None if lens is None else lens.data_ptr(), float(scale),
                                        _stream_ptr(stream)))

    def attend_fetched(self, layer: int, q: torch.Tensor, scale: float, out: torch.Tensor | None = None,
                       lse: torch.Tensor | None = None, lens: torch.Tensor | None = None, stream=None):
        """hs_attend_fetched: after fetch_misses and attend_resident, attend the misses and merge."""
        n_req = q.shape[0]
        if lens is not None:
            _require(lens.dtype == torch.int32 and lens.is_contiguous() and lens.dim() == 1 and lens.shape[0] >= n_req)
        out, lse = self._attn_io(q, out, lse)
        self._on_device(lens)
        _check(lib().hs_attend_fetched(self._h, layer, n_req, q.data_ptr(),
                                       None if lens is None else lens.data_ptr(), float(scale), out.data_ptr(),
                                       lse.data_ptr(), _stream_ptr(stream)))
        return out, lse

    # -- state -----------------------------------------------------------------------------------
    def state(self, layer: int) -> dict:
        """Torch views (no copies) of one layer's device tables and slot buffer."""
        v = StateView()
        _check(lib().hs_device_state(self._h, layer, ctypes.byref(v)))
        base = self.block.data_ptr()

        def view(ptr, count, dtype, shape):
            off = ptr - base
            esz = torch.empty(0, dtype=dtype).element_size()
            return self.block[off: off + count * esz].view(dtype).view(*shape)

        n, B, cap = self.n, self.B, v.capacity
        _require(v.request_stride == (B + 1) * v.slot_stride)
        rows = view(v.kv_buffer, n * v.request_stride, torch.uint8, (n, B + 1, v.slot_stride))
        return {
            "page_table": view(v.page_table, n * cap, torch.int32, (n, cap)),
            "slot_owner": view(v.slot_owner, n * B, torch.int32, (n, B)),
            "slot_stamp": view(v.slot_stamp, n * B, torch.int32, (n, B)),
            "lru_order": view(v.lru_order, n * B, torch.int32, (n, B)),
            "step": view(v.step, n, torch.int32, (n,)),
            "fresh_slots": view(v.fresh_slots, n * ((B + 31) // 32), torch.int32, (n, (B + 31) // 32)),
            # per request: B slot rows, then a row of zeros that padded attention entries read
            "kv_buffer": rows[:, :B],
            "zero_row": rows[:, B],
            "entry_bytes": v.entry_bytes,
            "page_tokens": v.page_tokens,
            "tail_plane": view(v.tail_plane, n * cap * v.tail_bytes, torch.uint8, (n, cap, v.tail_bytes))
            if v.tail_plane else None,
        }

    def reset_requests(self, first: int, count: int, stream=None):
        _check(lib().hs_reset_requests(self._h, first, count, _stream_ptr(stream)))

    def device_error(self) -> int:
        bits = ctypes.c_int32(0)
        _check(lib().hs_get_device_error(self._h, ctypes.byref(bits)))
        return bits.value
