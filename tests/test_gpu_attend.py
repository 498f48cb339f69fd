"""Sparse MLA decode attention on the GPU against the fp64 oracle.

Tolerance (max abs error): 2e-2 on the bf16 output -- the output is rounded to bf16 (relative
2^-9 of values below ~4.5) and P enters the MFMA as bf16 (relative 2^-9 per weight), while
products of bf16 q and decoded K are exact in fp32 and accumulate in fp32; lse, kept in fp32,
within 1e-3."""
import math

import numpy as np
import pytest
import torch

import hierarchical_kv_cache_hs_amd as hsa
import oracle
from synth import configs as C
from synth import kv as skv

from gpu_harness import Pair, say, trace_for

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

TOL_OUT = 2e-2
TOL_LSE = 1e-3
SCALE = 1.0 / math.sqrt(576)


def _bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def _compare(out_g, lse_g, out_o, lse_o, what):
    og = _bf16_to_f64(out_g)
    lg = lse_g.cpu().numpy().astype(np.float64)
    err = np.abs(og - out_o).max() if og.size else 0.0
    assert err <= TOL_OUT, f"{what}: max abs error {err}"
    fin = np.isfinite(lse_o)
    assert (np.isfinite(lg) == fin).all(), f"{what}: lse finiteness differs"
    if fin.any():
        lerr = np.abs(lg[fin] - lse_o[fin]).max()
        assert lerr <= TOL_LSE, f"{what}: lse error {lerr}"
    return err


def _attend_pair(p: Pair, layer, q_bits, slots, heads):
    q = torch.from_numpy(q_bits.view(np.int16)).cuda().view(torch.bfloat16)
    out, lse = p.hs.attend(layer, q, torch.from_numpy(slots).cuda(), SCALE)
    torch.cuda.synchronize()
    out_o, lse_o = p.orc.attend(layer, q_bits, slots, SCALE)
    return out, lse, out_o, lse_o


@pytest.mark.parametrize("layout", [hsa.LAYOUT_BF16, hsa.LAYOUT_FP8])
def test_tiny_every_step(layout):
    w = C.TINY.with_(layout=layout, n=2)
    say(f"attend tiny, layout {layout}: 2 requests, k 64, B 128, 32 steps")
    x = trace_for(w)
    p = Pair(w.n, 1, w.k, w.B, w.ratio, layout, w.seed, heads=16)
    worst = 0.0
    try:
        for t in range(x.shape[0]):
            slots, _ = p.step(0, x[t], check_state=False)
            qb = skv.queries(w.seed, t, w.n, 0, 16)
            out, lse, out_o, lse_o = _attend_pair(p, 0, qb, slots, 16)
            worst = max(worst, _compare(out, lse, out_o, lse_o, f"step {t}"))
            # exactness: same as attention over the host rows of the selected tokens
            o2, l2 = oracle.attend_rows(qb, x[t], p.orc.host[:, 0], layout, SCALE)
            assert np.abs(out_o - o2).max() < 1e-12
    finally:
        p.close()
    say(f"worst abs error {worst:.3e}")


@pytest.mark.parametrize("churn", C.FP8_256_CHURNS)
def test_fp8_256_full_size_sampled_steps(churn):
    """Every request's attention at steps 0 (all misses), 5 and 11 (steady state) of the
    256-request fp8 workload at each churn."""
    w = C.churn_point(churn)
    steps = 12
    say(f"attend fp8_256: 256 requests, k 2048, B 4096, churn {churn}, {steps} steps, attention at 0/5/11")
    x = trace_for(w, steps=steps)
    p = Pair(w.n, 1, w.k, w.B, w.ratio, w.layout, w.seed, heads=16)
    try:
        for t in range(steps):
            slots, _ = p.step(0, x[t], check_state=False)
            if t in (0, 5, steps - 1):
                qb = skv.queries(w.seed, t, w.n, 0, 16)
                out, lse, out_o, lse_o = _attend_pair(p, 0, qb, slots, 16)
                err = _compare(out, lse, out_o, lse_o, f"step {t}")
                say(f"step {t}: max abs error {err:.3e}")
    finally:
        p.close()


@pytest.mark.parametrize("layout,heads,k,B,n", [(hsa.LAYOUT_BF16, 16, 100, 160, 3), (hsa.LAYOUT_FP8, 5, 37, 64, 2),
                                                (hsa.LAYOUT_BF16, 1, 1, 4, 2), (hsa.LAYOUT_FP8, 16, 1000, 1024, 1),
                                                (hsa.LAYOUT_BF16, 16, 2048, 4096, 300)])
def test_ragged_shapes_and_padding(layout, heads, k, B, n):
    say(f"attend ragged: layout {layout}, heads {heads}, k {k}, B {B}, n {n}")
    rng = np.random.default_rng(k + heads)
    cap = 4 * B
    p = Pair(n, 1, k, B, 4, layout, seed=31, heads=heads)
    try:
        for t in range(3):
            S = np.stack([rng.choice(cap, k, replace=False) for _ in range(n)]).astype(np.int32)
            S[rng.random(S.shape) < 0.2] = -1
            if n > 1:
                S[1] = -1       # a request with no valid entry: out 0, lse -inf
            slots, _ = p.step(0, S, check_state=False)
            qb = skv.queries(31, t, n, 0, heads)
            out, lse, out_o, lse_o = _attend_pair(p, 0, qb, slots, heads)
            _compare(out, lse, out_o, lse_o, f"step {t}")
            if n > 1:
                assert (out[1].float() == 0).all() and torch.isneginf(lse[1]).all()
    finally:
        p.close()


def test_launch_sizes_below_the_handle_size():
    """Splits follow each launch's request count (n_req * splits within the 256 compute units):
    launches of 1, 17, 100, 129 and 200 requests on a 256-request handle, against the oracle."""
    n, k, B, heads = 256, 512, 1024, 16
    say("attend launch sizes: handle of 256 requests, launches of 1, 17, 100, 129, 200")
    rng = np.random.default_rng(77)
    p = Pair(n, 1, k, B, 2, hsa.LAYOUT_FP8, seed=53, heads=heads)
    try:
        S = np.stack([rng.choice(2 * B, k, replace=False) for _ in range(n)]).astype(np.int32)
        slots, _ = p.step(0, S, check_state=False)
        for nr in (1, 17, 100, 129, 200):
            qb = skv.queries(53, nr, nr, 0, heads)
            q = torch.from_numpy(qb.view(np.int16)).cuda().view(torch.bfloat16)
            out, lse = p.hs.attend(0, q, torch.from_numpy(slots[:nr]).cuda(), SCALE)
            torch.cuda.synchronize()
            out_o, lse_o = p.orc.attend(0, qb, slots[:nr], SCALE)
            _compare(out, lse, out_o, lse_o, f"{nr} requests")
    finally:
        p.close()


@pytest.mark.parametrize("layout", [hsa.LAYOUT_BF16, hsa.LAYOUT_FP8])
@pytest.mark.parametrize("n", [4, 300])
def test_trailing_padding(layout, n):
    """Selections valid only in a prefix (short contexts): requests with 0, 1, 63, 64, 65, 300 and
    all 2048 valid entries in one batch, one split and several; the tiles past the last valid
    entry are skipped, which must not change the result."""
    k, B, heads = 2048, 4096, 16
    say(f"attend trailing padding: layout {layout}, n {n}")
    rng = np.random.default_rng(5 + n + layout)
    p = Pair(n, 1, k, B, 2, layout, seed=43, heads=heads)
    try:
        S = np.stack([rng.choice(2 * B, k, replace=False) for _ in range(n)]).astype(np.int32)
        valid = [0, 1, 63, 64, 65, 300, k]
        for r in range(n):
            S[r, valid[r % len(valid)]:] = -1
        slots, _ = p.step(0, S, check_state=False)
        qb = skv.queries(43, 0, n, 0, heads)
        out, lse, out_o, lse_o = _attend_pair(p, 0, qb, slots, heads)
        _compare(out, lse, out_o, lse_o, "trailing padding")
        assert (out[0].float() == 0).all() and torch.isneginf(lse[0]).all()
    finally:
        p.close()


@pytest.mark.parametrize("layout,k,n", [(hsa.LAYOUT_FP8, 200, 3), (hsa.LAYOUT_BF16, 70, 2)])
def test_padding_ignores_nan_rows(layout, k, n):
    """Padded (-1) and out-of-range slot entries contribute nothing even when every slot that
    is not selected -- slot 0 included -- holds NaN bytes; the zero row after each request's
    slots is what padded entries read, and resolves never write it."""
    B = 256
    say(f"attend padding over NaN rows: layout {layout}, k {k}, B {B}, n {n}")
    rng = np.random.default_rng(7)
    hs = hsa.HiSparse(k, B, 2, n, 1, layout, num_heads=16)
    try:
        E = skv.ENTRY_BYTES[layout]
        rows = np.full((n, B, E), 0xFF, dtype=np.uint8)           # NaN in fp8 and bf16 alike
        slots = np.stack([rng.choice(np.arange(1, B), k, replace=False) for _ in range(n)]).astype(np.int32)
        for r in range(n):
            good = skv.rows_at(5, r, 0, np.arange(k), layout)
            rows[r, slots[r]] = good
        pad = rng.random(slots.shape) < 0.3
        slots[pad] = -1
        slots[0, :3] = [B, B + 7, -5]                             # out of range: treated as padding
        st = hs.state(0)
        st["kv_buffer"].copy_(torch.from_numpy(rows).cuda())
        assert not bool(st["zero_row"].any())
        qb = skv.queries(5, 0, n, 0, 16)
        q = torch.from_numpy(qb.view(np.int16)).cuda().view(torch.bfloat16)
        out, lse = hs.attend(0, q, torch.from_numpy(slots).cuda(), SCALE)
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
        idx = np.where((slots >= 0) & (slots < B), slots, -1)
        out_o, lse_o = oracle.attend_rows(qb, idx, rows, layout, SCALE)
        _compare(out, lse, out_o, lse_o, "padding over NaN rows")
        # resolves (row copies included) leave the zero rows untouched
        sel = torch.from_numpy(np.stack([rng.choice(4 * B // 2, k, replace=False) for _ in range(n)])
                               .astype(np.int32)).cuda()
        hs.resolve(0, sel)
        hs.resolve(0, sel, split=True)
        torch.cuda.synchronize()
        assert not bool(hs.state(0)["zero_row"].any())
    finally:
        hs.close()


def _decode_torch(rows: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(rows))
    lat = t[:, :512].contiguous().view(torch.float8_e4m3fn).to(torch.float64)
    sc = t[:, 512:528].contiguous().view(torch.float32).to(torch.float64)
    return (lat * sc.repeat_interleave(128, dim=1)).numpy()


@pytest.mark.parametrize("kind", ["normal", "subnormal"])
def test_fp8_every_code_decodes_exactly(kind):
    """One valid token per request: the output is that token's V row, exactly (power-of-two scales)."""
    say(f"attend fp8 every code ({kind})")
    finite = [c for c in range(256) if (c & 0x7F) != 0x7F]
    codes = np.array([c for c in finite if ((c & 0x78) == 0) == (kind == "subnormal")], dtype=np.uint8)
    scales = np.array([2.0 ** -7, 2.0 ** -6, 2.0 ** -8, 2.0 ** -7] if kind == "normal" else [2.0 ** 8] * 4,
                      np.float32)
    n, k, B = 8, 4, 8
    p = Pair(n, 1, k, B, 2, hsa.LAYOUT_FP8, seed=1, heads=16)
    try:
        rows = np.zeros((n, 656), np.uint8)
        for r in range(n):
            rows[r, :512] = np.roll(np.resize(codes, 512), 37 * r)
            rows[r, 512:528] = np.roll(scales, r).view(np.uint8)
            rows[r, 528:] = skv.rows_at(1, r, 0, [0], hsa.LAYOUT_FP8)[0, 528:]
            p.hs.host_kv(0, r)[5] = rows[r]
            p.orc.host[r, 0, 5] = rows[r]
        S = np.full((n, k), -1, np.int32)
        S[:, 2] = 5
        slots, _ = p.step(0, S, check_state=True)
        qb = skv.queries(2, 0, n, 0, 16)
        out, lse, out_o, lse_o = _attend_pair(p, 0, qb, slots, 16)
        V = _decode_torch(rows)
        got = _bf16_to_f64(out)
        for r in range(n):
            assert (got[r] == V[r][None, :]).all(), f"request {r}: decoded row differs"
            assert (out_o[r] == V[r][None, :]).all()
    finally:
        p.close()


def test_fp8_all_codes_mixed_rows():
    """All finite codes in attention over many tokens, with value magnitudes within a few units."""
    say("attend fp8 all codes, mixed")
    n, k, B = 1, 254, 256
    p = Pair(n, 1, k, B, 2, hsa.LAYOUT_FP8, seed=1, heads=16)
    try:
        codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
        host = p.hs.host_kv(0, 0)
        rows = np.zeros((k, 656), np.uint8)
        for i in range(k):
            rows[i, :512] = np.roll(np.resize(codes, 512), i)
            rows[i, 512:528] = (np.array([1.0, 0.5, 0.25, 0.75], np.float32) / 224).view(np.uint8)
            rows[i, 528:] = skv.rows_at(1, 0, 0, [i], hsa.LAYOUT_FP8)[0, 528:]
        host[:k] = rows
        p.orc.host[0, 0, :k] = rows
        S = np.arange(k, dtype=np.int32)[None]
        slots, _ = p.step(0, S, check_state=True)
        for t in range(3):
            qb = skv.queries(2, t, 1, 0, 16)
            out, lse, out_o, lse_o = _attend_pair(p, 0, qb, slots, 16)
            _compare(out, lse, out_o, lse_o, "all codes")
    finally:
        p.close()


def test_attend_graph_replay_matches_eager():
    say("attend in a captured graph, replayed")
    w = C.TINY.with_(n=4, layout=hsa.LAYOUT_FP8)
    x = trace_for(w)
    p = Pair(w.n, 1, w.k, w.B, w.ratio, w.layout, w.seed, heads=16)
    try:
        slots, _ = p.step(0, x[0], check_state=False)
        qb = skv.queries(w.seed, 0, w.n, 0, 16)
        q = torch.from_numpy(qb.view(np.int16)).cuda().view(torch.bfloat16)
        sl = torch.from_numpy(slots).cuda()
        out = torch.empty(w.n, 16, 512, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(w.n, 16, dtype=torch.float32, device="cuda")
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                p.hs.attend(0, q, sl, SCALE, out, lse, stream=s)
        torch.cuda.current_stream().wait_stream(s)
        e_out, e_lse = p.hs.attend(0, q, sl, SCALE)
        torch.cuda.synchronize()
        for i in range(4):
            out.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, e_out) and torch.equal(lse, e_lse), f"replay {i}"
    finally:
        p.close()


def test_attend_unsupported_without_heads():
    hs = hsa.HiSparse(8, 16, 2, 1)
    try:
        with pytest.raises(hsa.HSError):
            hs.attend(0, torch.zeros(1, 16, 576, dtype=torch.bfloat16, device="cuda"),
                      torch.zeros(1, 8, dtype=torch.int32, device="cuda"), 0.1)
    finally:
        hs.close()


def test_binding_refuses_mismatched_tensors():
    """The binding checks every tensor against the handle's sizes before anything is enqueued:
    a query with another head count, an undersized or wrongly typed lse, a CPU tensor or a
    slot array of the wrong width raise ValueError, and the output buffers stay untouched."""
    hs = hsa.HiSparse(8, 16, 2, 2, num_heads=16)
    try:
        dev = "cuda"
        q = torch.zeros(2, 16, 576, dtype=torch.bfloat16, device=dev)
        slots = torch.full((2, 8), -1, dtype=torch.int32, device=dev)
        out = torch.full((2, 16, 512), 7.0, dtype=torch.bfloat16, device=dev)
        lse = torch.full((2, 16), 7.0, dtype=torch.float32, device=dev)
        bad = [
            dict(q=torch.zeros(2, 8, 576, dtype=torch.bfloat16, device=dev)),     # 8 heads, handle 16
            dict(lse=torch.zeros(2, 8, dtype=torch.float32, device=dev)),         # undersized lse
            dict(lse=torch.zeros(2, 16, dtype=torch.float16, device=dev)),        # lse dtype
            dict(out=torch.zeros(2, 16, 512, dtype=torch.bfloat16)),              # out on the CPU
            dict(slots=torch.full((2, 4), -1, dtype=torch.int32, device=dev)),    # slots narrower than k
        ]
        for i, kw in enumerate(bad):
            args = dict(q=q, slots=slots, out=out, lse=lse)
            args.update(kw)
            with pytest.raises(ValueError):
                hs.attend(0, args["q"], args["slots"], SCALE, args["out"], args["lse"])
        torch.cuda.synchronize()
        assert (out.float() == 7.0).all() and (lse == 7.0).all(), "a refused call wrote its outputs"
        # the same buffers with matching shapes are accepted (all padding: out 0, lse -inf)
        hs.attend(0, q, slots, SCALE, out, lse)
        torch.cuda.synchronize()
        assert (out.float() == 0.0).all() and torch.isneginf(lse).all()
    finally:
        hs.close()
