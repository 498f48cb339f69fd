"""The seeded input generators: determinism, shape of the traces, row encodings."""
import numpy as np
import pytest
import torch

from synth import configs as C
from synth import kv as skv
from synth import trace as tr


def test_trace_deterministic_and_seed_sensitive():
    sp = C.TINY.trace_spec()
    a, b = tr.generate(sp), tr.generate(sp)
    assert a.tobytes() == b.tobytes()
    c = tr.generate(C.TINY.with_(index=7).trace_spec())
    assert a.tobytes() != c.tobytes()


@pytest.mark.parametrize("w", [C.TINY, C.BATCH64.with_(n=3, steps=30), C.FP8_256.with_(n=2, steps=40),
                               C.SWEEP.with_(n=2, steps=20), C.PAGES.with_(n=2, steps=40)])
def test_trace_shape(w):
    sp = w.trace_spec()
    x = tr.generate(sp)
    T, n, k = x.shape
    assert (T, n, k) == (sp.steps, sp.n, sp.k)
    h = sp.hist
    c = int(np.floor(sp.churn * h + 0.5))
    for r in range(n):
        prev = None
        for t in range(T):
            S = x[t, r]
            L_t = sp.ctx + (-(-t // w.page_tokens) if sp.grow else 0)   # units: tokens or pages
            assert len(set(S.tolist())) == k
            assert S.min() >= 0 and S.max() < L_t
            window = set(range(L_t - sp.window, L_t))
            assert window <= set(S.tolist())
            hist = set(S.tolist()) - window
            assert len(hist) == h and max(hist) < L_t - sp.window
            if prev is not None:
                # at most c history members replaced per step (a dropped one may be drawn back)
                assert len(hist - prev) <= c
            prev = hist
        # the emitted order is shuffled, not sorted
        assert not (np.diff(x[0, r]) > 0).all()


def test_page_trace_tracks_a_token_growing_context():
    # pages of P tokens over a context growing a token per step: at step t the context holds
    # len_tokens(t) tokens, the newest (partly written) page is ceil(len / P) - 1, and the
    # recency window always holds it
    w = C.PAGES.with_(n=3, steps=50)
    P = w.page_tokens
    x = tr.generate(w.trace_spec())
    for t in range(w.steps):
        L = w.len_tokens(t)
        assert L == w.ctx * P + t
        newest = -(-L // P) - 1
        assert (x[t].max(axis=1) == newest).all()
        assert all(newest in set(x[t, r].tolist()) for r in range(w.n))


def test_trace_prefix_is_stable():
    sp = C.BATCH64.with_(n=4, steps=12).trace_spec()
    full = tr.generate(sp)
    part = tr.generate(sp, steps=5, requests=2)
    assert (full[:5, :2] == part).all()


@pytest.mark.parametrize("layout", [skv.LAYOUT_BF16, skv.LAYOUT_FP8])
def test_c_rows_equal_numpy_restatement(layout):
    pos = [0, 1, 2, 77, 4095, 123456]
    a = skv.rows_at(1234, 5, 3, pos, layout)
    for i, p in enumerate(pos):
        assert (a[i] == skv.row_numpy(1234, 5, 3, p, layout)).all()
    big = np.empty((5000, skv.ENTRY_BYTES[layout]), np.uint8)
    skv.fill_rows(1234, 5, 3, 0, 5000, layout, big.ctypes.data, big.shape[1], nthreads=4)
    assert (big[[0, 1, 2, 77]] == a[:4]).all()


@pytest.mark.parametrize("layout,body", [(skv.LAYOUT_FP8, 640), (skv.LAYOUT_BF16, 1024), (skv.LAYOUT_FP8, 16)])
def test_split_rows_equal_whole_rows(layout, body):
    """The split writer (host part of each row at one stride, the rest at another, as the
    resident-tail layout stores them) writes exactly the whole rows' bytes, threaded or not."""
    E = skv.ENTRY_BYTES[layout]
    whole = np.empty((6000, E), np.uint8)
    skv.fill_rows(77, 2, 1, 300, 6000, layout, whole.ctypes.data, E, nthreads=4)
    head = np.full((6000, body + 32), 0xAB, np.uint8)          # a padded stride: the pad must stay
    tail = np.empty((6000, E - body), np.uint8)
    skv.fill_rows_split(77, 2, 1, 300, 6000, layout, head.ctypes.data, body + 32, body, tail.ctypes.data, E - body,
                        nthreads=4)
    assert (head[:, :body] == whole[:, :body]).all() and (head[:, body:] == 0xAB).all()
    assert (tail == whole[:, body:]).all()
    with pytest.raises(ValueError):
        skv.fill_rows_split(77, 2, 1, 0, 1, layout, head.ctypes.data, E, E, tail.ctypes.data, 16)


def test_normal_table_statistics():
    tb, tf = skv.normal_tables()
    assert abs(float(tf.mean())) < 1e-6 and abs(float(tf.std()) - 1.0) < 2e-3
    rows = skv.rows_at(3, 0, 0, np.arange(2000), skv.LAYOUT_BF16)
    v = skv.bf16_bits_to_f32(rows.view(np.uint16))
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1.0) < 0.01


def test_e4m3_encoder_matches_torch_rounding():
    # torch's float32 -> float8_e4m3fn conversion rounds to nearest even within range.
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(size=20000) * 100, rng.normal(size=20000) * 0.01,
                        np.array([0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, 0.0146484375])])
    x = np.clip(x, -448, 448).astype(np.float32)
    ours = skv.e4m3_encode_np(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch keeps the sign of zero, so compare values
    vo = torch.from_numpy(ours).view(torch.float8_e4m3fn).float().numpy()
    vr = torch.from_numpy(ref).view(torch.float8_e4m3fn).float().numpy()
    assert (vo == vr).all()
    lib = skv._lib()
    for v in x[::97]:
        assert lib.synth_e4m3_encode(float(v)) == skv.e4m3_encode_np(np.array([v], np.float32))[0] or v == 0


def test_fp8_rows_block_scales():
    rows = skv.rows_at(9, 1, 2, np.arange(50), skv.LAYOUT_FP8)
    codes = rows[:, :512]
    scales = rows[:, 512:528].copy().view(np.float32)
    assert (scales > 0).all()
    # every 128-block reaches the top code magnitude (amax maps to 448)
    mags = codes.reshape(50, 4, 128) & 0x7F
    assert (mags.max(axis=2) == 0x7E).all()


def test_queries_deterministic():
    a = skv.queries(1, 2, 3, 0, 16)
    b = skv.queries(1, 2, 3, 0, 16)
    c = skv.queries(1, 3, 3, 0, 16)
    assert a.shape == (3, 16, 576) and (a == b).all() and not (a == c).all()
