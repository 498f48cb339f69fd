"""The five synthetic workloads, with their shapes.

Each stands in for a serving situation the HiSparse pages describe: top-k 2048
selections, device buffers of 2048-6144 slots and host-to-device ratios of 8-10
(note, section 3), long contexts at high concurrency (note, section 1; paper
abstract), DSA-style MLA entries in bf16 or FP8 (GLM-5.1-FP8, note, section 1)
and models that share one selection across layers (paper abstract).  Where a
workload leaves a ratio open, ``cap = ceil(context_max / B) * B``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

from .kv import LAYOUT_BF16, LAYOUT_FP8, ENTRY_BYTES
from .trace import TraceSpec


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    n: int               # requests
    layers: int
    ctx: int
    k: int               # top_k
    B: int               # device_buffer_size (slots per request-layer)
    ratio: int           # host_to_device_ratio: host capacity = ratio * B tokens
    layout: int
    steps: int
    window: int
    zipf_s: float
    churn: float
    grow: bool
    attend: bool
    heads: int = 16
    shared_layers: bool = True
    description: str = ""
    page_tokens: int = 1   # tokens per selected unit; with P > 1, ctx, k, B, window count pages of P tokens

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def cap(self) -> int:
        return self.ratio * self.B

    @property
    def entry_bytes(self) -> int:
        return ENTRY_BYTES[self.layout]

    def trace_spec(self) -> TraceSpec:
        return TraceSpec(n=self.n, k=self.k, ctx=self.ctx, window=self.window, zipf_s=self.zipf_s,
                         churn=self.churn, steps=self.steps, grow=self.grow, seed=self.seed,
                         grow_per=self.page_tokens)

    def len_tokens(self, t: int) -> int:
        """Context length in tokens at step t (one new token per step when growing)."""
        return self.ctx * self.page_tokens + (t if self.grow else 0)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _ratio_for(ctx_max: int, B: int) -> int:
    return math.ceil(ctx_max / B)


TINY = Workload("tiny", 0, n=1, layers=1, ctx=4096, k=64, B=128, ratio=32, layout=LAYOUT_BF16, steps=32,
                window=16, zipf_s=1.1, churn=0.25, grow=False, attend=True,
                description="1 request, 1 layer, ctx 4096, bf16 576, k 64, B 128, 32 steps")

BATCH64 = Workload("batch64", 1, n=64, layers=1, ctx=32768, k=2048, B=4096, ratio=8, layout=LAYOUT_BF16,
                   steps=200, window=128, zipf_s=1.05, churn=0.10, grow=False, attend=False,
                   description="64 requests, 1 layer, ctx 32768, bf16 576 (1152 B), k 2048, B 4096, "
                               "ratio 8, 200 steps, resolve only")

FP8_256 = Workload("fp8_256", 2, n=256, layers=1, ctx=32768, k=2048, B=4096, ratio=9, layout=LAYOUT_FP8,
                   steps=200, window=128, zipf_s=1.05, churn=0.10, grow=True, attend=True,
                   description="256 requests, 1 layer, ctx 32768 + 1/step, fp8 656 B, k 2048, B 4096, "
                               "churn 2/10/30 %, resolve + MLA attention (16 heads)")
FP8_256_CHURNS = (0.02, 0.10, 0.30)

SWEEP = Workload("sweep", 3, n=32, layers=1, ctx=131072, k=2048, B=4096, ratio=32, layout=LAYOUT_BF16,
                 steps=100, window=256, zipf_s=1.0, churn=0.10, grow=False, attend=False,
                 description="32 requests, ctx 131072, bf16 1152 B, k 2048, B in {2048, 4096, 6144}, 100 steps")
SWEEP_BUFFERS = (2048, 4096, 6144)

PREFETCH = Workload("prefetch", 4, n=128, layers=8, ctx=65536, k=2048, B=4096, ratio=16, layout=LAYOUT_FP8,
                    steps=100, window=128, zipf_s=1.05, churn=0.10, grow=False, attend=True,
                    description="128 requests, 8 layers sharing a selection, ctx 65536, fp8 656 B, k 2048, "
                                "B 4096, layer-wise prefetch")

# Page-granular selections (paper abstract: the NSA and Quest families select blocks of
# tokens): Quest-sized pages of 16 tokens with the token budget of the fp8 workload --
# 128 pages = 2048 tokens selected, 256 pages = 4096 token rows of device buffer -- over a
# 32768-token context that grows a token per step, so the newest page is partly written.
PAGES = Workload("pages", 5, n=256, layers=1, ctx=2048, k=128, B=256, ratio=9, layout=LAYOUT_FP8,
                 steps=200, window=8, zipf_s=1.05, churn=0.10, grow=True, attend=True, page_tokens=16,
                 description="256 requests, pages of 16 tokens, ctx 32768 tokens + 1/step, fp8 656 B, "
                             "k 128 pages (2048 tokens), B 256 pages (4096 rows), resolve + MLA attention "
                             "cut at the context length (16 heads)")

ALL = (TINY, BATCH64, FP8_256, SWEEP, PREFETCH, PAGES)


def sweep_point(B: int) -> Workload:
    return SWEEP.with_(B=B, ratio=_ratio_for(SWEEP.ctx, B))


def churn_point(churn: float) -> Workload:
    return FP8_256.with_(churn=churn)
