"""hs_attend_noalloc -- the attention entry point that allocates nothing (its split partials live
in a static device array) -- against hs_attend through the C ABI, bit for bit on the same
handle and inputs: two calls in a row, the second with fewer requests, in both row layouts and
the fp32-output mode; on a resolve-only handle (no heads at creation) against a handle with
heads fed the same trace; and the refusal when a launch would need more partials than the array
holds.  The first call is also checked against the fp64 oracle at the usual tolerances."""
import ctypes
import math

import numpy as np
import pytest
import torch

import hierarchical_kv_cache_hs_amd as hsa

from gpu_harness import Pair, fill_host_pool, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

SCALE = 1.0 / math.sqrt(576)


def _selection(rng, n, cap, k):
    return np.stack([rng.choice(cap, k, replace=False) for _ in range(n)]).astype(np.int32)


def _q(rng, n, heads):
    return (torch.from_numpy(rng.standard_normal((n, heads, 576)).astype(np.float32)).to(torch.bfloat16)
            .contiguous().cuda())


def _noalloc(hs, layer, q, slots, out, lse):
    """The C entry point itself, with caller-allocated outputs."""
    st = hsa.lib().hs_attend_noalloc(hs.handle, layer, q.shape[0], q.shape[1], q.data_ptr(), slots.data_ptr(),
                                     ctypes.c_float(SCALE), out.data_ptr(), lse.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
    return st


@pytest.mark.parametrize("layout,flags", [(hsa.LAYOUT_FP8, 0), (hsa.LAYOUT_BF16, 0),
                                          (hsa.LAYOUT_FP8, hsa.FLAG_ATTN_OUT_F32)])
def test_noalloc_equals_attend_on_two_calls(layout, flags):
    n, k, B, ratio = 5, 1024, 1536, 4
    say(f"no-alloc attention: layout {layout}, flags {flags}, {n} then 3 requests, k {k}")
    rng = np.random.default_rng(71 + layout + flags)
    p = Pair(n, 1, k, B, ratio, layout, seed=71, heads=16, flags=flags)
    try:
        S = _selection(rng, n, ratio * B, k)
        S[1, 600:] = -1                                         # a padded request
        slots_np, _ = p.step(0, S, check_state=False)
        slots = torch.from_numpy(slots_np).cuda()
        q = _q(rng, n, 16)
        for m in (n, 3):                                        # second call: fewer requests
            out_a, lse_a = p.hs.attend(0, q[:m], slots[:m], SCALE)
            out_b = torch.full_like(out_a, float("nan"))
            lse_b = torch.full_like(lse_a, float("nan"))
            assert _noalloc(p.hs, 0, q[:m], slots[:m].contiguous(), out_b, lse_b) == hsa.HS_OK
            torch.cuda.synchronize()
            assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b), f"{m} requests: differs from hs_attend"
            if m == n:
                qb = q.cpu().view(torch.int16).numpy().view(np.uint16)
                out_o, lse_o = p.orc.attend(0, qb, slots_np, SCALE)
                tol = 1e-5 if flags & hsa.FLAG_ATTN_OUT_F32 else 2e-2
                assert np.abs(out_b.float().cpu().numpy() - out_o).max() <= tol
                assert np.abs(lse_b.cpu().numpy() - lse_o).max() <= (1e-5 if tol == 1e-5 else 1e-3)
    finally:
        p.close()


@pytest.mark.parametrize("heads", [16, 8])
def test_noalloc_on_a_resolve_only_handle(heads):
    """A handle created without heads reserves no partials; hs_attend_noalloc attends its rows
    anyway, equal to hs_attend on a handle with heads fed the same trace."""
    n, k, B, ratio, seed = 4, 512, 768, 4, 72
    say(f"no-alloc attention on a resolve-only handle: {heads} heads")
    rng = np.random.default_rng(seed + heads)
    a = hsa.HiSparse(k, B, ratio, n, 1, hsa.LAYOUT_FP8, 0, 0)
    b = hsa.HiSparse(k, B, ratio, n, 1, hsa.LAYOUT_FP8, heads, 0)
    try:
        fill_host_pool(a, seed)
        fill_host_pool(b, seed)
        with pytest.raises(hsa.HSError):                         # hs_attend needs heads at creation
            a.attend(0, _q(rng, n, heads), torch.zeros(n, k, dtype=torch.int32, device="cuda"), SCALE)
        for t in range(3):
            sel = torch.from_numpy(_selection(rng, n, ratio * B, k)).cuda()
            sa, ma = a.resolve(0, sel)
            sb, mb = b.resolve(0, sel)
            q = _q(rng, n, heads)
            out_b, lse_b = b.attend(0, q, sb, SCALE)
            out_a, lse_a = a.attend_noalloc(0, q, sa, SCALE)
            torch.cuda.synchronize()
            assert torch.equal(sa, sb) and torch.equal(ma, mb)
            assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b), f"step {t}"
    finally:
        a.close()
        b.close()


def test_noalloc_refuses_launches_beyond_its_array():
    """200 requests of 4096 fp8 tokens take two workgroups each: 400 partials > 256."""
    say("no-alloc attention: refusal beyond the static array")
    n, k = 200, 4096
    h = hsa.HiSparse(k, k, 1, n, 1, hsa.LAYOUT_FP8, 0, hsa.FLAG_NO_IO)
    try:
        q = torch.zeros(n, 16, 576, dtype=torch.bfloat16, device="cuda")
        slots = torch.full((n, k), -1, dtype=torch.int32, device="cuda")
        out = torch.empty(n, 16, 512, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(n, 16, dtype=torch.float32, device="cuda")
        assert _noalloc(h, 0, q, slots, out, lse) == hsa.HS_ERR_UNSUPPORTED
        assert "256" in hsa.lib().hs_last_error_message().decode()
        assert _noalloc(h, 0, q[:1], slots[:1], out[:1], lse[:1]) == hsa.HS_OK   # 1 x 16 partials
        torch.cuda.synchronize()
        assert torch.isinf(lse[:1]).all() and (out[:1].float() == 0).all()      # every entry padding
    finally:
        h.close()
