"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

* The CPU oracle (oracle/hs_oracle.c) is rebuilt with -fsanitize=address,undefined and the
  oracle pin tests run against that build in a child process (libasan preloaded, UB fatal).
* The library's host API (hs_api.cpp: configuration checks, memory plans, argument checks,
  handle creation and release) is built with a host compiler and the same sanitizers, with
  host stand-ins for the device launches (tests/host_stubs.cpp), and driven through the C ABI
  with valid, invalid and NULL arguments: plans of every layout, rejected configurations,
  a creation that fails at the first HIP call (no GPU here) and releases its handle, and
  every entry point's argument checks.

Any report from either sanitizer aborts the child and fails the test."""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hierarchical_kv_cache_hs_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="needs gcc and g++")


def _asan_runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not path or not os.path.exists(path):
        pytest.skip("libasan is not available")
    return path


def _child_env(extra):
    env = dict(os.environ)
    env.update({"LD_PRELOAD": _asan_runtime(),
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
                "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
                "PYTHONPATH": ROOT, "CUDA_VISIBLE_DEVICES": "", "HIP_VISIBLE_DEVICES": ""})
    env.update(extra)
    return env


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    lib = tmp_path / "liboracle_san.so"
    subprocess.check_call(["gcc", *SAN, "-std=c11", "-fPIC", "-shared", "-pthread", "-o", str(lib),
                           os.path.join(ROOT, "oracle", "hs_oracle.c"), "-lm"])
    pins = [os.path.join(ROOT, "tests", f) for f in ("test_oracle_pins.py", "test_oracle_append_pins.py",
                                                      "test_oracle_policy_pins.py", "test_oracle_page_pins.py")]
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *pins],
                         env=_child_env({"HS_ORACLE_LIB": str(lib)}), capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail


def test_host_api_under_asan_and_ubsan(tmp_path):
    lib = tmp_path / "libhs_host_san.so"
    subprocess.check_call(["g++", *SAN, "-std=c++17", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
                           "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                           "-o", str(lib), os.path.join(CSRC, "hs_api.cpp"),
                           os.path.join(ROOT, "tests", "host_stubs.cpp"),
                           "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64"])
    script = textwrap.dedent(f"""
        import ctypes, sys
        sys.path.insert(0, {ROOT!r})
        import hierarchical_kv_cache_hs_amd as hsa
        L = ctypes.CDLL({str(lib)!r})
        p, i32, f = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float(1.0)
        for name in ("hs_device_bytes", "hs_host_bytes"):
            getattr(L, name).argtypes = [ctypes.POINTER(hsa.Config), ctypes.POINTER(ctypes.c_size_t)]
        L.hs_create.argtypes = [ctypes.POINTER(hsa.Config), ctypes.POINTER(p)]
        L.hs_last_error_message.restype = ctypes.c_char_p
        L.hs_status_string.restype = ctypes.c_char_p
        n = ctypes.c_size_t()
        ok = [dict(top_k=64, device_buffer_size=128, host_to_device_ratio=32, max_requests=1),
              dict(top_k=2048, device_buffer_size=4096, host_to_device_ratio=16, max_requests=128, num_layers=8,
                   layout=1, num_heads=16),
              dict(top_k=128, device_buffer_size=256, host_to_device_ratio=9, max_requests=4, layout=1, num_heads=16,
                   page_tokens=16),
              dict(top_k=8192, device_buffer_size=16384, host_to_device_ratio=2, max_requests=2, flags=3),
              dict(top_k=2048, device_buffer_size=4096, host_to_device_ratio=16, max_requests=128, num_layers=8,
                   layout=1, num_heads=16, flags=4)]
        bad = [dict(top_k=0, device_buffer_size=8, host_to_device_ratio=1, max_requests=1),
               dict(top_k=9, device_buffer_size=8, host_to_device_ratio=1, max_requests=1),
               dict(top_k=8, device_buffer_size=8, host_to_device_ratio=0, max_requests=1),
               dict(top_k=8, device_buffer_size=8, host_to_device_ratio=1, max_requests=1, layout=7),
               dict(top_k=8, device_buffer_size=8, host_to_device_ratio=1, max_requests=1, num_heads=17),
               dict(top_k=8, device_buffer_size=8, host_to_device_ratio=1, max_requests=1, flags=0x80),
               dict(top_k=8, device_buffer_size=8, host_to_device_ratio=1, max_requests=1, page_tokens=3),
               dict(top_k=8, device_buffer_size=8, host_to_device_ratio=1, max_requests=1, flags=4),
               dict(top_k=8, device_buffer_size=8, host_to_device_ratio=1 << 30, max_requests=1 << 30),
               dict(top_k=1 << 20, device_buffer_size=1 << 20, host_to_device_ratio=1, max_requests=1)]
        for kw in ok:
            c = hsa.make_config(**kw)
            assert L.hs_device_bytes(ctypes.byref(c), ctypes.byref(n)) == 0 and n.value > 0
            assert L.hs_host_bytes(ctypes.byref(c), ctypes.byref(n)) == 0
            h = p()
            st = L.hs_create(ctypes.byref(c), ctypes.byref(h))   # no GPU: fails at the first HIP call
            assert st != 0 and not h.value, st
            assert L.hs_last_error_message()
        for kw in bad:
            c = hsa.make_config(**kw)
            assert L.hs_device_bytes(ctypes.byref(c), ctypes.byref(n)) != 0 and n.value == 0
            h = p()
            assert L.hs_create(ctypes.byref(c), ctypes.byref(h)) in (1, 3) and not h.value
            assert L.hs_last_error_message()
        assert L.hs_create(None, None) == 1 and L.hs_device_bytes(None, None) == 1
        for s in range(-1, 8):
            assert L.hs_status_string(s)
        assert L.hs_destroy(None) == 0
        bits = ctypes.c_int32()
        assert L.hs_get_device_error(None, ctypes.byref(bits)) == 1
        assert L.hs_resolve(None, 0, 1, None, None, None, None) == 1
        assert L.hs_resolve_tables(None, 0, 1, None, None, None, None) == 1
        assert L.hs_fetch_misses(None, 0, 1, None) == 1
        assert L.hs_attend(None, 0, 1, None, None, f, None, None, None) == 1
        assert L.hs_attend_pages(None, 0, 1, None, None, None, None, f, None, None, None) == 1
        assert L.hs_attend_noalloc(None, 0, 1, 16, None, None, f, None, None, None) == 1
        assert L.hs_attend_resident(None, 0, 1, None, None, None, None, f, None) == 1
        assert L.hs_attend_fetched(None, 0, 1, None, None, f, None, None, None) == 1
        assert L.hs_append(None, 0, 1, None, None, ctypes.c_int64(656), None, None) == 1
        assert L.hs_offload(None, 0, 0, ctypes.c_int64(0), ctypes.c_int64(1), None, ctypes.c_int64(656), None) == 1
        assert L.hs_topk(None, 1, None, ctypes.c_int64(4), None, None, None) == 1
        assert L.hs_topk_hinted(None, 1, None, ctypes.c_int64(4), None, None, None, None) == 1
        assert L.hs_host_kv(None, 0, 0, None, None, None) == 1
        assert L.hs_device_state(None, 0, None) == 1
        assert L.hs_reset_requests(None, 0, 1, None) == 1
        assert L.hs_stream_read(None, 16, None, None) == 1
        print("host api ok")
    """)
    res = subprocess.run([sys.executable, "-c", script], env=_child_env({}), capture_output=True, text=True,
                         timeout=300)
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0 and "host api ok" in res.stdout, tail
