"""Top-k selection from indexer scores on the GPU (hs_topk) against the oracle, bit-exact:
random and tie-heavy scores, every length regime (0, < k, = k, > k, ragged), -inf, +-0,
long contexts, range errors; then the chain into the resolver with a different selection per
layer, eager and captured in a graph."""
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


def _run(hs, s, lens):
    sel = hs.topk(torch.from_numpy(s).cuda(), torch.from_numpy(lens.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    return sel.cpu().numpy()


@pytest.mark.parametrize("k,stride,n,kind", [(64, 4096, 5, "normal"), (64, 4096, 5, "ties"),
                                             (2048, 32768, 3, "normal"), (2048, 32768, 3, "ties"),
                                             (1, 100, 4, "ties"), (7, 8, 6, "ties"), (2048, 131072, 2, "normal"),
                                             (500, 20000, 4, "specials")])
def test_topk_matches_oracle(k, stride, n, kind):
    say(f"topk: k {k}, stride {stride}, n {n}, {kind}")
    rng = np.random.default_rng(k + stride + len(kind))
    B = max(k, 8)
    hs = hsa.HiSparse(k, B, (stride + B - 1) // B, n, 1, hsa.LAYOUT_BF16)
    try:
        for rep in range(3):
            if kind == "normal":
                s = rng.standard_normal((n, stride)).astype(np.float32)
            elif kind == "ties":
                s = rng.integers(-4, 5, size=(n, stride)).astype(np.float32)
            else:
                s = rng.standard_normal((n, stride)).astype(np.float32)
                s[rng.random((n, stride)) < 0.2] = -np.inf
                s[rng.random((n, stride)) < 0.2] = 0.0
                s[rng.random((n, stride)) < 0.2] = -0.0
                s[rng.random((n, stride)) < 0.05] = np.float32(3.4e38)
            lens = rng.integers(0, stride + 1, size=n)
            lens[0] = stride
            if n > 1:
                lens[1] = min(k, stride)
            if n > 2:
                lens[2] = max(0, k - 1)
            got = _run(hs, s, lens)
            want = topk_oracle(s, lens, k)
            assert (got == want).all(), f"rep {rep}: differs from the oracle"
        assert hs.device_error() == 0
    finally:
        hs.close()


@pytest.mark.parametrize("plant", ["small", "large", "equal"])
@pytest.mark.parametrize("stride,k", [(65536, 2048), (20000, 500), (8192, 8000)])
def test_topk_rows_with_planted_values(plant, stride, k):
    """Rows with a planted score at every position floor(i n / 4096), i < min(n, 4096): a
    value far below the rest (the top-k avoids them), far above it (they fill the top of the
    selection, or all of it), or one shared value (a digit full of ties); full and shortened
    rows, k up to 8000 of 8192.  Bit-exact against the oracle."""
    say(f"topk planted values: k {k}, stride {stride}, planted {plant}")
    rng = np.random.default_rng(stride + k + len(plant))
    n = 4
    B = max(k, 8)
    hs = hsa.HiSparse(k, B, (stride + B - 1) // B, n, 1, hsa.LAYOUT_BF16)
    try:
        s = rng.standard_normal((n, stride)).astype(np.float32)
        lens = np.array([stride, stride - 7, max(k + 1, stride // 2), k + 1])
        value = {"small": -3.0e38, "large": 3.0e38, "equal": 0.25}[plant]
        for r in range(n):
            m = int(lens[r])
            S = min(m, 4096)
            pos = (np.arange(S, dtype=np.int64) * m) // S
            s[r, pos] = value
        got = _run(hs, s, lens)
        want = topk_oracle(s, lens, k)
        assert (got == want).all(), "differs from the oracle"
        assert hs.device_error() == 0
    finally:
        hs.close()


def test_topk_length_out_of_range_sets_error():
    k, stride = 16, 64
    hs = hsa.HiSparse(k, 16, 2, 2, 1, hsa.LAYOUT_BF16)           # capacity 32 < stride
    try:
        s = np.arange(2 * stride, dtype=np.float32).reshape(2, stride)
        got = _run(hs, s, np.array([33, 20]))
        assert (got[0] == -1).all()
        assert (got[1] == topk_oracle(s[1:], np.array([20]), k)[0]).all()
        assert hs.device_error() & hsa.DEVERR_TOKEN_RANGE
        with pytest.raises(hsa.HSError):
            hs.topk(torch.zeros(2, 30, device="cuda"), torch.zeros(2, dtype=torch.int32, device="cuda"))
    finally:
        hs.close()


@pytest.mark.parametrize("graph", [False, True])
def test_topk_feeds_resolver_with_per_layer_selections(graph):
    """Synthetic indexer scores -> top-k -> resolve, a different selection per layer; tables,
    slots and misses match the oracle chain bit for bit."""
    n, L, k, B, ctx, W, seed = 4, 3, 256, 512, 8192, 32, 21
    say(f"topk -> resolve: n {n}, layers {L}, k {k}, B {B}, ctx {ctx}, graph {graph}")
    hs = hsa.HiSparse(k, B, ctx // B, n, L, hsa.LAYOUT_BF16)
    orc = oracle.OracleCache(n, L, B, ctx)
    lens_d = torch.full((n,), ctx, dtype=torch.int32, device="cuda")
    scores_d = torch.empty(L, n, ctx, dtype=torch.float32, device="cuda")
    sel_d = torch.empty(L, n, k, dtype=torch.int32, device="cuda")
    slots_d = torch.empty(L, n, k, dtype=torch.int32, device="cuda")
    miss_d = torch.empty(L, n, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()

    def step():
        for l in range(L):
            hs.topk(scores_d[l], lens_d, sel_d[l], stream=stream)
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
        for t in range(6):
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
                slots_o, miss_o = orc.resolve(l, want_sel)
                assert (slots_d[l].cpu().numpy() == slots_o).all(), f"step {t} layer {l}: slots"
                assert (miss_d[l].cpu().numpy() == miss_o).all()
                st = hs.state(l)
                assert (st["page_table"].cpu().numpy() == orc.PT[:, l]).all()
                assert (st["slot_stamp"].cpu().numpy().astype(np.int64) == orc.ST[:, l]).all()
            if t > 0:                                   # layers select differently
                assert not np.array_equal(sel_d[0].cpu().numpy(), sel_d[1].cpu().numpy())
    finally:
        hs.close()


@pytest.mark.parametrize("k,stride", [(2048, 65536), (64, 4096), (500, 20000)])
def test_topk_whole_digit_taken(k, stride):
    """Rows where the k largest keys fill whole digits of the radix select: exactly k positions
    planted with one large value (the first digit holds exactly the k needed keys), and k
    positions planted with distinct values that share their top 24 bits, with and without 50
    lower keys in the same first digit (then the second digit holds exactly the k), over N(0,1)
    scores.  Bit-exact against the oracle."""
    say(f"topk whole digits: k {k}, stride {stride}")
    rng = np.random.default_rng(k + stride)
    n = 3
    hs = hsa.HiSparse(k, max(k, 8), (stride + max(k, 8) - 1) // max(k, 8), n, 1, hsa.LAYOUT_BF16)
    try:
        s = rng.standard_normal((n, stride)).astype(np.float32)
        lens = np.array([stride, stride - 5, stride // 2])
        for r in range(n):
            pos = rng.choice(int(lens[r]), size=k, replace=False)
            if r == 0:
                s[r, pos] = np.float32(1000.0)
            else:
                # distinct floats with equal top 24 key bits: 1000.0 plus small mantissa steps
                base = np.float32(1000.0).view(np.uint32)
                s[r, pos] = (base + np.arange(k, dtype=np.uint32) % 200).view(np.float32)
            if r == 2:
                # and 50 keys of 999.0 (the same top 12 key bits, lower next 12): the first digit
                # then holds more than k keys and the second one exactly k
                rest = np.setdiff1d(np.arange(int(lens[r])), pos)
                s[r, rng.choice(rest, size=50, replace=False)] = np.float32(999.0)
        got = _run(hs, s, lens)
        want = topk_oracle(s, lens, k)
        assert (got == want).all(), "differs from the oracle"
        assert hs.device_error() == 0
    finally:
        hs.close()
