"""hs_topk_hinted on the GPU: the selection must equal the oracle's (and hs_topk's) bit for bit
for any hint -- none, right, one digit off (still inside the bracket), two or more off, the
extremes, random -- on random, tie-heavy and special-value rows and every length regime; the
hint written back must be the top 12 bits of the order key of the k-th largest score (-1 when
every position is selected or the row is rejected); and hints carried across the steps of a
decode loop, eager and captured in a graph, keep the chain into the resolver equal to the
oracle's."""
import numpy as np
import pytest
import torch

import hierarchical_kv_cache_hs_amd as hsa
import oracle
from oracle.topk import topk as topk_oracle
from synth import scores as sc

from gpu_harness import say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]


def order_key(x: np.ndarray) -> np.ndarray:
    """The documented key of a score: unsigned order = float order, -0 joined with +0."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    k = np.where(b & 0x80000000, ~b & 0xFFFFFFFF, b | 0x80000000)
    return np.where(b == 0x80000000, k + 1, k).astype(np.uint64)


def expected_hint(s: np.ndarray, lens: np.ndarray, want: np.ndarray, k: int) -> np.ndarray:
    """Top 12 key bits of the k-th largest score of each row (its smallest selected score)."""
    out = np.full(s.shape[0], -1, dtype=np.int64)
    for r in range(s.shape[0]):
        if lens[r] > k:
            kth = s[r, want[r]].min()
            out[r] = int(order_key(np.array([kth]))[0] >> 20)
    return out


def _rows(kind, rng, n, stride):
    if kind == "normal":
        return rng.standard_normal((n, stride)).astype(np.float32)
    if kind == "ties":
        return rng.integers(-4, 5, size=(n, stride)).astype(np.float32)
    s = rng.standard_normal((n, stride)).astype(np.float32)
    s[rng.random((n, stride)) < 0.2] = -np.inf
    s[rng.random((n, stride)) < 0.2] = 0.0
    s[rng.random((n, stride)) < 0.2] = -0.0
    s[rng.random((n, stride)) < 0.05] = np.float32(3.4e38)
    return s


@pytest.mark.parametrize("k,stride,n,kind", [(2048, 65536, 6, "normal"), (64, 4096, 6, "ties"),
                                             (500, 20000, 6, "specials"), (2048, 32768, 6, "ties"),
                                             (7, 8, 6, "normal"), (8000, 8192, 6, "normal")])
def test_hinted_selection_equals_oracle_for_any_hint(k, stride, n, kind):
    say(f"topk hinted: k {k}, stride {stride}, n {n}, {kind}")
    rng = np.random.default_rng(3 * k + stride + len(kind))
    B = max(k, 8)
    hs = hsa.HiSparse(k, B, (stride + B - 1) // B, n, 1, hsa.LAYOUT_BF16)
    try:
        for rep in range(3):
            s = _rows(kind, rng, n, stride)
            lens = rng.integers(k + 1 if stride > k else 0, stride + 1, size=n)
            lens[0] = stride
            lens[n - 1] = min(k, stride)                      # every position selected
            want = topk_oracle(s, lens, k)
            hint_true = expected_hint(s, lens, want, k)
            base = np.where(hint_true >= 0, hint_true, 2048)
            guesses = {
                "none": np.full(n, -1),
                "right": base,
                "one below": base - 1,
                "one above": base + 1,
                "two below": base - 2,
                "two above": base + 2,
                "extremes": np.where(np.arange(n) % 2 == 0, 0, 4095),
                "random": rng.integers(-3, 4100, size=n),
            }
            s_d = torch.from_numpy(s).cuda()
            lens_d = torch.from_numpy(lens.astype(np.int32)).cuda()
            for name, g in guesses.items():
                hint = torch.from_numpy(np.clip(g, -5, 5000).astype(np.int32)).cuda()
                sel = hs.topk(s_d, lens_d, hint=hint)
                torch.cuda.synchronize()
                assert (sel.cpu().numpy() == want).all(), f"rep {rep}, guess {name}: selection differs"
                assert (hint.cpu().numpy() == hint_true).all(), f"rep {rep}, guess {name}: hint written back"
        assert hs.device_error() == 0
    finally:
        hs.close()


def test_hinted_rejects_bad_rows_and_null_hint():
    n, k, stride = 3, 16, 64
    hs = hsa.HiSparse(k, k, 2, n, 1, hsa.LAYOUT_BF16)      # capacity 32 tokens
    try:
        s = torch.randn(n, stride, device="cuda")
        lens = torch.tensor([20, 40, 5], dtype=torch.int32, device="cuda")   # 40 > capacity
        hint = torch.full((n,), 7, dtype=torch.int32, device="cuda")
        sel = hs.topk(s, lens, hint=hint)
        torch.cuda.synchronize()
        got = sel.cpu().numpy()
        assert (got[1] == -1).all() and (hint.cpu().numpy()[1:] == -1).all()
        assert hs.device_error() & hsa.DEVERR_TOKEN_RANGE
        want = topk_oracle(s.cpu().numpy(), np.array([20, 0, 5]), k)
        assert (got[0] == want[0]).all() and (got[2] == want[2]).all()
        L = hsa.lib()
        assert L.hs_topk_hinted(hs.handle, n, s.data_ptr(), stride, lens.data_ptr(), sel.data_ptr(), None,
                                None) == hsa.HS_ERR_INVALID_ARG
    finally:
        hs.close()


@pytest.mark.parametrize("graph", [False, True])
def test_hinted_decode_loop_feeds_resolver(graph):
    """Synthetic indexer scores of 8 steps -> hinted top-k (one hint per layer, carried from
    step to step) -> resolve, a different selection per layer: selections, slots, misses and
    tables equal the oracle chain; the hints equal the true digits after every step."""
    n, L, k, B, ctx, W, seed = 8, 3, 2048, 4096, 65536, 128, 33
    say(f"topk hinted -> resolve: n {n}, layers {L}, k {k}, ctx {ctx}, graph {graph}")
    hs = hsa.HiSparse(k, B, ctx // B, n, L, hsa.LAYOUT_FP8, flags=hsa.FLAG_NO_IO)
    orc = oracle.OracleCache(n, L, B, ctx, layout=hsa.LAYOUT_FP8)
    lens_d = torch.full((n,), ctx, dtype=torch.int32, device="cuda")
    scores_d = torch.empty(L, n, ctx, dtype=torch.float32, device="cuda")
    sel_d = torch.empty(L, n, k, dtype=torch.int32, device="cuda")
    slots_d = torch.empty(L, n, k, dtype=torch.int32, device="cuda")
    miss_d = torch.empty(L, n, dtype=torch.int32, device="cuda")
    hints = torch.full((L, n), -1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()

    def step():
        for l in range(L):
            hs.topk(scores_d[l], lens_d, sel_d[l], stream=stream, hint=hints[l])
            hs.resolve(l, sel_d[l], slots_d[l], miss_d[l], stream=stream)

    try:
        g = None
        if graph:
            g = torch.cuda.CUDAGraph()
            stream.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(stream):
                with torch.cuda.graph(g, stream=stream):
                    step()
            torch.cuda.synchronize()
            hints.fill_(-1)                         # the capture did not run
            hs.reset_requests(0, n)
            torch.cuda.synchronize()
        for t in range(8):
            s = np.stack([sc.batch(seed, n, l, t, ctx, W, ctx) for l in range(L)])
            scores_d.copy_(torch.from_numpy(s))
            torch.cuda.synchronize()
            with torch.cuda.stream(stream):
                if graph:
                    g.replay()
                else:
                    step()
            torch.cuda.synchronize()
            for l in range(L):
                want_sel = topk_oracle(s[l], np.full(n, ctx), k)
                assert (sel_d[l].cpu().numpy() == want_sel).all(), f"step {t} layer {l}: selection"
                assert (hints[l].cpu().numpy() == expected_hint(s[l], np.full(n, ctx), want_sel, k)).all()
                slots_o, miss_o = orc.resolve(l, want_sel)
                assert (slots_d[l].cpu().numpy() == slots_o).all(), f"step {t} layer {l}: slots"
                assert (miss_d[l].cpu().numpy() == miss_o).all()
            st = hs.state(L - 1)
            assert (st["page_table"].cpu().numpy() == orc.PT[:, L - 1]).all()
    finally:
        hs.close()


def _key_float(k: int) -> np.float32:
    """The score whose order key is k (non-NaN keys 0x007FFFFF .. 0xFF800000)."""
    bits = (k ^ 0x80000000) if (k & 0x80000000) else (~k & 0xFFFFFFFF)
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


@pytest.mark.parametrize("sign", [1, -1])
def test_scores_on_digit_edges(sign):
    """Rows whose scores sit on, one key below and one key above the top-digit edges around the
    k-th largest score (the bracket's bounds and the plain pass's digit bounds are compared
    against such floats), with a few hundred ties at the k-th largest: the k-th largest lies on
    an edge, one key above it, or (rows 3 ..) one key below it.  Plain and hinted selections
    and the returned digit equal the oracle's for hints at the true digit, one off and two off."""
    n, k, B, stride = 6, 4000, 4096, 8192
    say(f"topk digit edges: sign {sign}, k {k}, stride {stride}")
    rng = np.random.default_rng(77 + sign)
    hs = hsa.HiSparse(k, B, stride // B, n, 1, hsa.LAYOUT_BF16)
    try:
        mid = 0xBF8 if sign > 0 else 0x407                    # digit of +1.0 / of -1.125
        s = np.empty((n, stride), dtype=np.float32)
        for r in range(n):
            keys = [(d << 20) + o for d in range(mid - 3, mid + 4) for o in (-1, 0, 1)]
            if r >= 3:    # no key on or above the middle digit's lower edge: its top one below
                keys = [kk for kk in keys if not (kk >> 20 == mid and kk & 0xFFFFF <= 1)]
            edges = np.array([_key_float(kk) for kk in keys], dtype=np.float32)
            pick = rng.integers(0, edges.size, size=stride)
            s[r] = edges[pick]
            spread = rng.random(stride) < 0.3
            s[r, spread] = (edges[pick[spread]] * np.float32(1 + 0.01 * rng.standard_normal(spread.sum()))).astype(np.float32)
        lens = np.full(n, stride)
        lens[1] = stride - 5                                   # ragged tail
        want = topk_oracle(s, lens, k)
        hint_true = expected_hint(s, lens, want, k)
        s_d = torch.from_numpy(s).cuda()
        lens_d = torch.from_numpy(lens.astype(np.int32)).cuda()
        sel = hs.topk(s_d, lens_d)
        torch.cuda.synchronize()
        assert (sel.cpu().numpy() == want).all(), "plain selection"
        for delta in (0, -1, 1, -2, 2):
            hint = torch.from_numpy((hint_true + delta).astype(np.int32)).cuda()
            sel = hs.topk(s_d, lens_d, hint=hint)
            torch.cuda.synchronize()
            assert (sel.cpu().numpy() == want).all(), f"hint off by {delta}: selection"
            assert (hint.cpu().numpy() == hint_true).all(), f"hint off by {delta}: digit written back"
        assert hs.device_error() == 0
    finally:
        hs.close()
