"""The fp32-output attention mode (HS_FLAG_ATTN_OUT_F32) against the fp64 oracle, within the
1e-5 tier.

Tolerance (max abs error, output and lse): 1e-5.  Products of bf16 q and decoded K are exact
in fp32 and accumulate in fp32 (a score's error is a few fp32 roundings of terms of order 1);
P enters the P V product as three bf16 terms whose sum equals P to 2^-27 relative; the
output is a convex combination of values below ~5 in magnitude, so fp32 rounding of the sums
contributes a few 1e-7.  The bf16-output tier is tests/test_gpu_attend.py."""
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

TOL = 1e-5
SCALE = 1.0 / math.sqrt(576)
F32 = hsa.FLAG_ATTN_OUT_F32


def _compare(out_g, lse_g, out_o, lse_o, what):
    assert out_g.dtype == torch.float32
    og = out_g.cpu().numpy().astype(np.float64)
    lg = lse_g.cpu().numpy().astype(np.float64)
    err = np.abs(og - out_o).max() if og.size else 0.0
    assert err <= TOL, f"{what}: max abs error {err}"
    fin = np.isfinite(lse_o)
    assert (np.isfinite(lg) == fin).all(), f"{what}: lse finiteness differs"
    lerr = np.abs(lg[fin] - lse_o[fin]).max() if fin.any() else 0.0
    assert lerr <= TOL, f"{what}: lse error {lerr}"
    return err, lerr


def _q(qb):
    return torch.from_numpy(qb.view(np.int16)).cuda().view(torch.bfloat16)


@pytest.mark.parametrize("layout", [hsa.LAYOUT_BF16, hsa.LAYOUT_FP8])
def test_tiny_every_step_f32(layout):
    w = C.TINY.with_(layout=layout, n=2)
    say(f"attend f32 tiny, layout {layout}: 2 requests, k 64, B 128, 32 steps")
    x = trace_for(w)
    p = Pair(w.n, 1, w.k, w.B, w.ratio, layout, w.seed, heads=16, flags=F32)
    worst = 0.0
    try:
        for t in range(x.shape[0]):
            slots, _ = p.step(0, x[t], check_state=False)
            qb = skv.queries(w.seed, t, w.n, 0, 16)
            out, lse = p.hs.attend(0, _q(qb), torch.from_numpy(slots).cuda(), SCALE)
            out_o, lse_o = p.orc.attend(0, qb, slots, SCALE)
            torch.cuda.synchronize()
            worst = max(worst, _compare(out, lse, out_o, lse_o, f"step {t}")[0])
    finally:
        p.close()
    say(f"worst abs error {worst:.3e}")


@pytest.mark.parametrize("layout,heads,k,B,n", [(hsa.LAYOUT_BF16, 16, 100, 160, 3), (hsa.LAYOUT_FP8, 5, 37, 64, 2),
                                                (hsa.LAYOUT_BF16, 1, 1, 4, 2), (hsa.LAYOUT_FP8, 16, 2048, 4096, 1),
                                                (hsa.LAYOUT_BF16, 16, 2048, 4096, 300)])
def test_ragged_shapes_splits_and_padding_f32(layout, heads, k, B, n):
    say(f"attend f32 ragged: layout {layout}, heads {heads}, k {k}, B {B}, n {n}")
    rng = np.random.default_rng(k + heads + 1)
    cap = 4 * B
    p = Pair(n, 1, k, B, 4, layout, seed=37, heads=heads, flags=F32)
    try:
        for t in range(2):
            S = np.stack([rng.choice(cap, k, replace=False) for _ in range(n)]).astype(np.int32)
            S[rng.random(S.shape) < 0.2] = -1
            if n > 1:
                S[1] = -1
            slots, _ = p.step(0, S, check_state=False)
            qb = skv.queries(37, t, n, 0, heads)
            out, lse = p.hs.attend(0, _q(qb), torch.from_numpy(slots).cuda(), SCALE)
            out_o, lse_o = p.orc.attend(0, qb, slots, SCALE)
            torch.cuda.synchronize()
            err, lerr = _compare(out, lse, out_o, lse_o, f"step {t}")
            say(f"step {t}: out {err:.2e}, lse {lerr:.2e}")
            if n > 1:
                assert (out[1] == 0).all() and torch.isneginf(lse[1]).all()
    finally:
        p.close()


def test_fp8_256_full_size_sampled_f32():
    w = C.FP8_256
    steps = 6
    say(f"attend f32 fp8_256: 256 requests, k 2048, B 4096, {steps} steps, attention at 0 and {steps - 1}")
    x = trace_for(w, steps=steps)
    p = Pair(w.n, 1, w.k, w.B, w.ratio, w.layout, w.seed, heads=16, flags=F32)
    try:
        for t in range(steps):
            slots, _ = p.step(0, x[t], check_state=False)
            if t in (0, steps - 1):
                qb = skv.queries(w.seed, t, w.n, 0, 16)
                out, lse = p.hs.attend(0, _q(qb), torch.from_numpy(slots).cuda(), SCALE)
                out_o, lse_o = p.orc.attend(0, qb, slots, SCALE)
                torch.cuda.synchronize()
                err, lerr = _compare(out, lse, out_o, lse_o, f"step {t}")
                say(f"step {t}: out {err:.2e}, lse {lerr:.2e}")
    finally:
        p.close()


def test_pages_cut_f32():
    P, k, B, n, heads = 16, 40, 80, 3, 16
    say(f"attend_pages f32: P {P}, k {k}, B {B}, n {n}")
    rng = np.random.default_rng(5)
    p = Pair(n, 1, k, B, 4, hsa.LAYOUT_FP8, seed=41, heads=heads, flags=F32, page_tokens=P)
    try:
        for t in range(3):
            S = np.stack([rng.choice(4 * B, k, replace=False) for _ in range(n)]).astype(np.int32)
            S[rng.random(S.shape) < 0.1] = -1
            slots, _ = p.step(0, S, check_state=False)
            lens = rng.integers(1, 4 * B * P + 1, size=n).astype(np.int32)
            qb = skv.queries(41, t, n, 0, heads)
            out, lse = p.hs.attend_pages(0, _q(qb), torch.from_numpy(slots).cuda(), torch.from_numpy(S).cuda(),
                                         torch.from_numpy(lens).cuda(), SCALE)
            out_o, lse_o = p.orc.attend_pages(0, qb, slots, S, lens, SCALE)
            torch.cuda.synchronize()
            _compare(out, lse, out_o, lse_o, f"step {t}")
    finally:
        p.close()


def test_f32_mode_agrees_with_bf16_mode():
    """Both modes on the same handle state: the bf16 output is the fp32 output within the bf16 tier."""
    n, k, B, heads = 4, 512, 1024, 16
    say("attend f32 vs bf16 mode")
    rng = np.random.default_rng(9)
    a = hsa.HiSparse(k, B, 4, n, 1, hsa.LAYOUT_FP8, heads)
    b = hsa.HiSparse(k, B, 4, n, 1, hsa.LAYOUT_FP8, heads, F32)
    try:
        for hs in (a, b):
            for r in range(n):
                ptr, cap, stride = hs.host_kv_ptr(0, r)
                skv.fill_rows(3, r, 0, 0, cap, hsa.LAYOUT_FP8, ptr, stride)
        S = torch.from_numpy(np.stack([rng.choice(4 * B, k, replace=False) for _ in range(n)]).astype(np.int32)).cuda()
        sa, _ = a.resolve(0, S)
        sb, _ = b.resolve(0, S)
        q = _q(skv.queries(3, 0, n, 0, heads))
        oa, la = a.attend(0, q, sa, SCALE)
        ob, lb = b.attend(0, q, sb, SCALE)
        torch.cuda.synchronize()
        assert oa.dtype == torch.bfloat16 and ob.dtype == torch.float32
        assert (oa.float() - ob).abs().max().item() <= 2e-2
        assert (la - lb).abs().max().item() <= 1e-3
    finally:
        a.close()
        b.close()
