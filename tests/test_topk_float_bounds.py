"""The top-k kernel's candidate pass compares raw scores against float bounds instead of mapping
every score to its order key: "key(x) >= K" must equal "x >= bound(K)" for every score x (no
NaN) and every digit edge K = d * 2^20 (lower edges d = 0 .. 4095, upper edges d = 1 .. 4096, where
4096 wraps to 0 = no upper edge).  The
bound is the float whose key is K; edges at or below the key of -inf (0x007FFFFF, which only
-inf and NaN patterns lie below) take -inf; an upper edge of 2^32 and edges past +inf's key
take NaN, which no comparison passes.  This is checked exhaustively over the edges against
the documented key mapping, for scores at, next to and far from every edge and the special
values."""
import numpy as np


def order_key(x: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    k = np.where(b & 0x80000000, ~b & 0xFFFFFFFF, b | 0x80000000)
    return np.where(b == 0x80000000, k + 1, k).astype(np.uint64)


def key_float(k: int) -> np.float32:
    bits = (k ^ 0x80000000) if (k & 0x80000000) else (~k & 0xFFFFFFFF)
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


def lower_bound(k: int) -> np.float32:
    """The kernel's bound for "key >= k" as a lower edge (k < 2^32)."""
    return np.float32(-np.inf) if k <= 0x007FFFFF else key_float(k)


def upper_bound(k: int) -> np.float32:
    """The kernel's bound for "key >= k" as an upper edge: k == 0 stands for 2^32 (nothing)."""
    if k == 0:
        return np.float32(np.nan)
    return np.float32(-np.inf) if k <= 0x007FFFFF else key_float(k)


def _scores():
    special = [0.0, -0.0, np.inf, -np.inf, np.finfo(np.float32).max, -np.finfo(np.float32).max,
               np.finfo(np.float32).tiny, -np.finfo(np.float32).tiny, 1e-45, -1e-45, 1.0, -1.0, 2.0, 1.875]
    near = []
    for d in range(4097):
        for k in (d << 20, (d << 20) - 1, (d << 20) + 1):
            if 0x007FFFFF <= k <= 0xFF800000:           # keys of non-NaN floats
                near.append(key_float(k))
    rng = np.random.default_rng(0)
    rand = rng.standard_normal(2000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 2000)
    x = np.concatenate([np.array(special, dtype=np.float32), np.array(near, dtype=np.float32),
                        rand.astype(np.float32)])
    return x[~np.isnan(x)]


def test_float_bounds_select_exactly_the_key_ranges():
    x = _scores()
    keys = order_key(x)
    with np.errstate(invalid="ignore"):
        for d in range(4097):
            k = (d << 20) & 0xFFFFFFFF
            if d < 4096:
                want = keys >= k
                assert (want == (x >= lower_bound(k))).all(), f"lower edge {d}"
            if d > 0:                                   # an upper edge is dhi + 1 >= 1
                want_up = keys >= (d << 20) if d < 4096 else np.zeros_like(keys, dtype=bool)
                assert (want_up == (x >= upper_bound(k))).all(), f"upper edge {d}"


def test_digit_ranges_partition_the_scores():
    """A bracket [dlo, dhi] built from the bounds holds exactly the scores whose key digit lies
    in it, and 'above' exactly those beyond it: together with the rest they partition x."""
    x = _scores()
    dig = (order_key(x) >> 20).astype(np.int64)
    with np.errstate(invalid="ignore"):
        for h in (0, 1, 2, 7, 8, 9, 1000, 2047, 2048, 3070, 3071, 4087, 4088, 4094, 4095):
            dlo, dhi = max(h - 1, 0), min(h + 1, 4095)
            hi = upper_bound(((dhi + 1) << 20) & 0xFFFFFFFF)
            lo = lower_bound(dlo << 20)
            above = x >= hi
            inside = (x >= lo) & ~above
            assert (above == (dig > dhi)).all(), f"hint {h}: above"
            assert (inside == ((dig >= dlo) & (dig <= dhi))).all(), f"hint {h}: inside"
