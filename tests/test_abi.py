"""The C ABI library: it loads, exports every function include/hs.h declares, and rejects
bad configurations on the host before any HIP call (runs without a GPU)."""
import ctypes
import os
import re

import pytest

import hierarchical_kv_cache_hs_amd as hsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "hs.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hs_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("hs_create", "hs_resolve", "hs_attend", "hs_destroy"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = hsa.lib()
    for n in _declared():
        assert hasattr(L, n), n
    assert set(_declared()) == set(hsa.SYMBOLS)


def _cfg(**kw):
    base = dict(top_k=64, device_buffer_size=128, host_to_device_ratio=32, max_requests=2, num_layers=1,
                layout=hsa.LAYOUT_BF16, num_heads=16, flags=0)
    base.update(kw)
    return hsa.make_config(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(top_k=0), hsa.HS_ERR_INVALID_ARG),
    (dict(device_buffer_size=63), hsa.HS_ERR_INVALID_ARG),
    (dict(host_to_device_ratio=0), hsa.HS_ERR_INVALID_ARG),
    (dict(max_requests=0), hsa.HS_ERR_INVALID_ARG),
    (dict(num_layers=0), hsa.HS_ERR_INVALID_ARG),
    (dict(layout=7), hsa.HS_ERR_INVALID_ARG),
    (dict(num_heads=17), hsa.HS_ERR_INVALID_ARG),
    (dict(num_heads=-1), hsa.HS_ERR_INVALID_ARG),
    (dict(flags=0x80), hsa.HS_ERR_INVALID_ARG),
    (dict(eviction=3), hsa.HS_ERR_INVALID_ARG),
    (dict(eviction=-1), hsa.HS_ERR_INVALID_ARG),
    (dict(top_k=8193, device_buffer_size=9000), hsa.HS_ERR_UNSUPPORTED),
    (dict(device_buffer_size=16385), hsa.HS_ERR_UNSUPPORTED),
    (dict(device_buffer_size=4096, host_to_device_ratio=600000), hsa.HS_ERR_INVALID_ARG),
    (dict(device_buffer_size=4096, host_to_device_ratio=300), hsa.HS_ERR_UNSUPPORTED),
    (dict(page_tokens=3), hsa.HS_ERR_INVALID_ARG),
    (dict(page_tokens=-4), hsa.HS_ERR_INVALID_ARG),
    (dict(page_tokens=512), hsa.HS_ERR_INVALID_ARG),
    (dict(top_k=2048, device_buffer_size=2048, page_tokens=64), hsa.HS_ERR_UNSUPPORTED),   # 131072 tokens
    (dict(device_buffer_size=16384, host_to_device_ratio=1, page_tokens=256), hsa.HS_ERR_UNSUPPORTED),  # > 4 GiB
    (dict(device_buffer_size=4096, host_to_device_ratio=4096, page_tokens=256), hsa.HS_ERR_INVALID_ARG),  # 2^32 tokens
    # the resident tail needs token-granular 656-byte rows and a host pool
    (dict(flags=hsa.FLAG_RESIDENT_TAIL, layout=hsa.LAYOUT_BF16), hsa.HS_ERR_INVALID_ARG),
    (dict(flags=hsa.FLAG_RESIDENT_TAIL, layout=hsa.LAYOUT_FP8, page_tokens=16), hsa.HS_ERR_INVALID_ARG),
    (dict(flags=hsa.FLAG_RESIDENT_TAIL | hsa.FLAG_NO_IO, layout=hsa.LAYOUT_FP8), hsa.HS_ERR_INVALID_ARG),
])
def test_create_rejects_bad_config_before_hip(kw, status):
    cfg = _cfg(**kw)
    h = ctypes.c_void_p(123)
    assert hsa.lib().hs_create(ctypes.byref(cfg), ctypes.byref(h)) == status
    assert h.value is None
    assert hsa.lib().hs_last_error_message().decode() != ""
    n = ctypes.c_size_t(7)
    assert hsa.lib().hs_device_bytes(ctypes.byref(cfg), ctypes.byref(n)) == status
    assert n.value == 0


def test_sizes_for_the_batch64_workload():
    cfg = _cfg(top_k=2048, device_buffer_size=4096, host_to_device_ratio=8, max_requests=64, num_heads=0)
    dev = hsa.device_bytes(cfg)
    host = hsa.host_bytes(cfg)
    assert host == 64 * 32768 * 1152
    slots = 64 * (4096 + 1) * 1152  # each request's slot rows and its zero row
    tables = 64 * 32768 * 4 + 3 * 64 * 4096 * 4 + 2 * 64 * 2048 * 4  # page table, owners/stamps/order, miss lists
    assert slots + tables <= dev <= slots + tables + 64 * 1024


def test_fp32_output_flag_is_accepted():
    assert hsa.device_bytes(_cfg(flags=hsa.FLAG_ATTN_OUT_F32)) == hsa.device_bytes(_cfg())
    assert hsa.device_bytes(_cfg(flags=hsa.FLAG_ATTN_OUT_F32 | hsa.FLAG_NO_IO)) > 0


def test_no_io_mode_has_no_host_pool():
    assert hsa.host_bytes(_cfg(flags=hsa.FLAG_NO_IO)) == 0
    assert hsa.host_bytes(_cfg()) == 2 * 128 * 32 * 1152


def test_page_sizes():
    # pages of 16: 256 slots of 16 rows, 32 pages of history per slot; the host pool keeps a row per token
    cfg = _cfg(top_k=128, device_buffer_size=256, host_to_device_ratio=8, max_requests=4, num_heads=0,
               layout=hsa.LAYOUT_FP8, page_tokens=16)
    assert hsa.host_bytes(cfg) == 4 * 256 * 8 * 16 * 656
    slots = 4 * (256 + 1) * 16 * 656
    tables = 4 * 2048 * 4 + 3 * 4 * 256 * 4 + 2 * 4 * 128 * 4
    assert slots + tables <= hsa.device_bytes(cfg) <= slots + tables + 64 * 1024
    tok = _cfg(top_k=128, device_buffer_size=256, host_to_device_ratio=8, max_requests=4, num_heads=0,
               layout=hsa.LAYOUT_FP8, page_tokens=1)
    assert hsa.device_bytes(_cfg(top_k=128, device_buffer_size=256, host_to_device_ratio=8, max_requests=4,
                                 num_heads=0, layout=hsa.LAYOUT_FP8, page_tokens=0)) == hsa.device_bytes(tok)


def test_resident_tail_sizes():
    # 656-byte rows: the host pool keeps 640 bytes per token row, the device adds 16 bytes per
    # token of history (the tail plane) to the packed layout's block
    kw = dict(top_k=128, device_buffer_size=256, host_to_device_ratio=8, max_requests=4, num_heads=16,
              layout=hsa.LAYOUT_FP8, num_layers=3)
    packed, tail = _cfg(**kw), _cfg(flags=hsa.FLAG_RESIDENT_TAIL, **kw)
    assert hsa.host_bytes(packed) == 3 * 4 * 2048 * 656
    assert hsa.host_bytes(tail) == 3 * 4 * 2048 * 640
    plane = 3 * 4 * 2048 * 16
    assert plane <= hsa.device_bytes(tail) - hsa.device_bytes(packed) <= plane + 256


def test_null_arguments():
    L = hsa.lib()
    assert L.hs_destroy(None) == hsa.HS_OK
    assert L.hs_resolve(None, 0, 1, None, None, None, None) == hsa.HS_ERR_INVALID_ARG
    assert L.hs_attend(None, 0, 1, None, None, ctypes.c_float(1.0), None, None, None) == hsa.HS_ERR_INVALID_ARG
    assert L.hs_attend_pages(None, 0, 1, None, None, None, None, ctypes.c_float(1.0), None, None,
                             None) == hsa.HS_ERR_INVALID_ARG
    assert L.hs_create(None, None) == hsa.HS_ERR_INVALID_ARG
    bits = ctypes.c_int32()
    assert L.hs_get_device_error(None, ctypes.byref(bits)) == hsa.HS_ERR_INVALID_ARG
    for s in range(6):
        assert L.hs_status_string(s)


def test_new_entry_points_reject_bad_arguments_before_hip():
    L = hsa.lib()
    f = ctypes.c_float(1.0)
    assert L.hs_attend_resident(None, 0, 1, None, None, None, None, f, None) == hsa.HS_ERR_INVALID_ARG
    assert L.hs_attend_fetched(None, 0, 1, None, None, f, None, None, None) == hsa.HS_ERR_INVALID_ARG
    assert L.hs_attend_noalloc(None, 0, 1, 16, None, None, f, None, None, None) == hsa.HS_ERR_INVALID_ARG
    assert L.hs_topk_hinted(None, 1, None, 4, None, None, None, None) == hsa.HS_ERR_INVALID_ARG
    sink = ctypes.c_uint32()
    assert L.hs_stream_read(None, 16, ctypes.byref(sink), None) == hsa.HS_ERR_INVALID_ARG
    buf = (ctypes.c_uint8 * 64)()
    base = ctypes.addressof(buf)
    aligned = (base + 15) & ~15
    assert L.hs_stream_read(aligned, 24, ctypes.byref(sink), None) == hsa.HS_ERR_INVALID_ARG   # not a multiple of 16
    assert L.hs_stream_read(aligned + 4, 16, ctypes.byref(sink), None) == hsa.HS_ERR_INVALID_ARG  # misaligned
    assert L.hs_stream_read(aligned, 16, None, None) == hsa.HS_ERR_INVALID_ARG
    assert L.hs_stream_read(aligned, 0, ctypes.byref(sink), None) == hsa.HS_OK                  # nothing to read
    assert hsa.lib().hs_last_error_message().decode() != ""

