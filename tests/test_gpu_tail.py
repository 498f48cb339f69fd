"""Resolver parity with the resident-tail layout (HS_FLAG_RESIDENT_TAIL): the host pool keeps
the first 640 bytes of each 656-byte row and the device keeps the last 16 in a tail plane.
Slots, miss counts, every table and the bytes of every occupied slot must equal the oracle's
(which knows only whole rows) bit for bit, on the fused resolve (with and without the early
host reads, 1024- and 512-thread workgroups) and on the list-only resolve + row copy."""
import numpy as np
import pytest
import torch

import hierarchical_kv_cache_hs_amd as hsa
from synth import configs as C
from synth import kv as skv

from gpu_harness import Pair, say, trace_for

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

TAIL = hsa.FLAG_RESIDENT_TAIL


# 64 requests: fused with early host reads (1024 threads); 128: without them; 256: the
# 512-thread fused workgroup
@pytest.mark.parametrize("split", [False, True], ids=["fused", "split"])
@pytest.mark.parametrize("requests", [64, 128, 256])
def test_fp8_256_resident_tail(requests, split):
    w = C.churn_point(0.10)
    steps = 30
    say(f"resident tail: {requests} requests of fp8_256 (churn 0.1), {steps} steps, split {split}")
    x = trace_for(w, steps=steps, requests=requests)
    p = Pair(requests, 1, w.k, w.B, w.ratio, w.layout, w.seed, flags=TAIL, oracle_rows=False, split=split)
    try:
        for t in range(steps):
            p.step(0, x[t], check_state=False)
            if t % 10 == 0 or t == steps - 1:
                p.check_state(0, requests, rows=True)      # every occupied slot's bytes
        say(f"{steps} steps: tables and every occupied slot match the oracle")
        # resolves only read the history: the tail plane still holds the generated tails
        pos = np.arange(w.cap)
        for r in (0, requests - 1):
            tails = p.hs.tail_plane(0)[r].cpu().numpy()
            assert (tails == skv.rows_at(w.seed, r, 0, pos, w.layout)[:, 640:]).all(), f"request {r}: tails"
        assert p.hs.device_error() == 0
    finally:
        p.close()


@pytest.mark.parametrize("k,B,ratio,n,split", [(700, 1000, 3, 3, False), (1, 7, 5, 2, False), (33, 33, 4, 5, False),
                                                (4096, 6000, 2, 2, False), (700, 1000, 3, 3, True),
                                                (1, 7, 5, 2, True), (4096, 6000, 2, 2, True)])
def test_resident_tail_ragged_shapes(k, B, ratio, n, split):
    say(f"resident tail ragged: k {k}, B {B}, ratio {ratio}, n {n}, split {split}")
    cap = B * ratio
    rng = np.random.default_rng(k * 5 + B)
    p = Pair(n, 1, k, B, ratio, hsa.LAYOUT_FP8, seed=91, flags=TAIL, split=split)
    try:
        pop = rng.permutation(cap)
        wt = 1.0 / np.arange(1, cap + 1) ** 0.9
        wt /= wt.sum()
        for t in range(10):
            S = np.stack([rng.choice(pop, k, replace=False, p=wt) for _ in range(n)]).astype(np.int32)
            S[rng.random(S.shape) < 0.05] = -1
            if t == 4:
                S[0] = -1          # a row of padding only
            p.step(0, S, check_state=True)
    finally:
        p.close()


def test_resident_tail_equals_packed_handle():
    """The same trace through a packed handle and a resident-tail handle: slots, misses and
    the slot buffers are equal byte for byte, over several layers."""
    w = C.PREFETCH.with_(n=5, ctx=8192, ratio=2)
    steps = 6
    x = trace_for(w, steps=steps)
    say(f"packed vs resident tail: {w.n} requests, {w.layers} layers, {steps} steps")
    a = Pair(w.n, w.layers, w.k, w.B, w.ratio, w.layout, w.seed, oracle_rows=False)
    b = Pair(w.n, w.layers, w.k, w.B, w.ratio, w.layout, w.seed, flags=TAIL, oracle_rows=False, split=True)
    try:
        for t in range(steps):
            for l in range(w.layers):
                sa, ma = a.step(l, x[t], check_state=False)
                sb, mb = b.step(l, x[t], check_state=False)
                assert (sa == sb).all() and (ma == mb).all()
        for l in range(w.layers):
            assert torch.equal(a.hs.state(l)["kv_buffer"], b.hs.state(l)["kv_buffer"]), f"layer {l}: slot bytes"
    finally:
        a.close()
        b.close()
