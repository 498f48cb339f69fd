"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle's checks.

This package holds input generation only (selection traces, KV rows, queries)
and none of the cache method's arithmetic.  Neither the device library nor the
oracle imports it; the callers hand its arrays to both.
"""
from . import kv, trace, configs  # noqa: F401
