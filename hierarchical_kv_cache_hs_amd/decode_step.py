"""A whole decode step over every layer, captured in one hipGraph.

For each layer l the step resolves the layer's selection (hit detection, LRU
replacement, table update, host-to-device fetch) and then runs sparse attention
over the resolved slots.  With ``prefetch=True`` the layers' resolves run back to
back on a second stream and each attention waits only for its own layer's
resolve, so resolving (and fetching) layer l + 1 overlaps attention of layer l; the table
resolves run on their own stream, ahead of the row copies, so the copies follow one another.
With ``split_attention=True`` as well, each layer's attention is split by residency: the
part over the resident tokens waits only for the layer's tables and runs beside the copies,
the part over the fetched misses waits for the layer's copy, so after the last layer's copy
only that part remains.  ``split_last=m`` splits only the last m layers' attention (the copy
kernel keeps attention workgroups off its compute units, so a resident part beside a copy
runs at its own pace on the other units).
This is valid when the layers share one selection known at the start of the step
(HiSparse paper abstract: exact layer-wise prefetching for models that share
selections across layers); the results are the same as the serial order because
layers own disjoint tables, slots and scratch.

Everything inside the graph is a libhs kernel launch; torch provides the streams,
events and buffers.
"""
from __future__ import annotations

import torch

from . import HiSparse


def attend_while_fetching(hs: HiSparse, layer: int, sel, q, scale: float, slots, miss, out, lse, main, side,
                          lens=None):
    """One layer of a decode step whose attention of the resident tokens overlaps the copy of
    the misses: list-only resolve on ``main``; the miss copy on ``side``; on ``main`` meanwhile
    the attention of the entries that were hits (their slots are not written by the copy);
    then, once both are done, the attention of the fetched misses and the merge into ``out`` /
    ``lse``.  With ``lens`` the attention is cut at each request's context length
    (hs_attend_pages semantics).  Enqueue-only: usable inside a graph capture."""
    n = sel.shape[0]
    hs.resolve_tables(layer, sel, slots, miss, stream=main)
    # the copy is enqueued (and in a graph, captured) first, so that its few workgroups are
    # placed before the attention's fill the compute units (256 requests of fp8 rows: 505
    # against 515 us per step with the attention enqueued first)
    side.wait_stream(main)                       # fork: the copy needs only the miss lists
    hs.fetch_misses(layer, n, stream=side)
    hs.attend_resident(layer, q, slots, scale, sel if lens is not None else None, lens, stream=main)
    main.wait_stream(side)                       # join: the misses have landed
    hs.attend_fetched(layer, q, scale, out, lse, lens=lens, stream=main)


def copy_waits(layers: int) -> dict:
    """{copy l: the last layer whose tables it waits for}, for row copies that follow one
    another on one stream while the tables of every layer run in layer order on another.

    Each cross-stream edge into a copy costs the graph ~5 us between consecutive copies, and
    the tables run far ahead of the copies, so only copies 0, 1, 2, 4, 8, ... wait: copy l for
    the tables of the layers up to 2l - 1 (copy 0 for its own), and each copy up to the next
    waiting one is covered (128 requests x 8 layers: 2.057 against 2.072 ms per step with a wait
    before every copy).  Waiting for every layer before copy 1 was slower: beside a copy and an
    attention a table resolve can take most of a copy's time."""
    out = {}
    for l in range(layers):
        if l == 0:
            out[0] = 0
        elif l & (l - 1) == 0:
            out[l] = min(2 * l - 1, layers - 1)
    return out


class DecodeSteps:
    """Captures ``len(sels)`` consecutive decode steps of ``hs`` into one graph.

    sels:  list of int32 [n][top_k] device tensors, one shared selection per step
    qs:    list of bf16 [L][n][H][576] device tensors, the queries of each step
    Outputs of the last replayed step are left in ``slots``, ``out`` and ``lse``;
    ``miss[i][l][r]`` records every step's miss counts.
    """

    def __init__(self, hs: HiSparse, sels, qs, scale: float, prefetch: bool, attend: bool = True,
                 split_attention: bool = False, capture: bool = True, split_last: int = 0):
        """With ``capture=False`` nothing is captured: :meth:`run_eager` enqueues the same
        launches, in the same stream order, one step at a time (used to time single kernels of
        the schedule with HIP events, which a captured graph does not expose).  With
        ``split_last=m`` (layer-wise prefetch only) the attention of the last m layers is split
        by residency: their resident parts run beside the last row copies, so that after the
        step's last copy only the attention of that layer's misses remains."""
        assert len(sels) == len(qs) and len(sels) > 0
        assert not split_attention or (prefetch and attend)
        split_last = int(split_last)
        assert 0 <= split_last <= hs.L
        assert not split_last or (prefetch and attend and not split_attention)
        self.hs, self.prefetch, self.attend, self.split_attention = hs, prefetch, attend, split_attention
        self.split_last = split_last
        self.fetch_events = None   # run_eager(time_fetches=True): (start, end) per fetch launch
        n = sels[0].shape[0]
        L, k = hs.L, hs.top_k
        dev = sels[0].device
        H = qs[0].shape[2]
        self.slots = torch.empty(L, n, k, dtype=torch.int32, device=dev)
        self.miss = torch.zeros(len(sels), L, n, dtype=torch.int32, device=dev)
        self.out = torch.empty(L, n, H, 512, dtype=hs.out_dtype, device=dev)
        self.lse = torch.empty(L, n, H, dtype=torch.float32, device=dev)
        self.stream = torch.cuda.Stream(device=dev)
        self.side = torch.cuda.Stream(device=dev)    # table resolves
        self.copy = torch.cuda.Stream(device=dev)    # row copies
        self.sels, self.qs, self.scale = sels, qs, scale
        self.graph = None
        if capture:
            self.graph = torch.cuda.CUDAGraph()
            self.stream.wait_stream(torch.cuda.current_stream(dev))
            with torch.cuda.stream(self.stream):
                with torch.cuda.graph(self.graph, stream=self.stream):
                    for i, (sel, q) in enumerate(zip(sels, qs)):
                        self._one_step(i, sel, q, scale)
            torch.cuda.current_stream(dev).wait_stream(self.stream)

    def run_eager(self, time_fetches: bool = False):
        """Enqueues every step without a graph (same kernels, streams and waits as the captured
        schedule).  With ``time_fetches`` (layer-wise prefetch with the copies on a stream of
        their own) each step's row-copy launches are bracketed by timing events on that stream,
        one before the first copy and one after the last, and the copies wait once for all the
        step's table resolves (which run ahead of them anyway) instead of once per layer, so
        they follow one another with no cross-stream wait in between; ``fetch_events`` then
        holds one (start, end) pair per step."""
        dev = self.slots.device
        self.fetch_events = [] if time_fetches else None
        self.stream.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(self.stream):
            for i, (sel, q) in enumerate(zip(self.sels, self.qs)):
                self._one_step(i, sel, q, self.scale)
        torch.cuda.current_stream(dev).wait_stream(self.stream)

    def _one_step(self, i, sel, q, scale):
        hs, main = self.hs, self.stream
        if not self.prefetch:
            for l in range(hs.L):
                hs.resolve(l, sel, self.slots[l], self.miss[i, l], stream=main)
                if self.attend:
                    hs.attend(l, q[l], self.slots[l], scale, self.out[l], self.lse[l], stream=main)
            return
        # Attention on the main stream.  With one attention per layer, the table resolves run
        # on one side stream and the row copies on another: the tables of layer l + 1 (a short,
        # latency-bound kernel) run while the rows of layer l are copied, so the link does not
        # idle between layers (128 requests x 8 layers: 2.16 against 2.23-2.28 ms).  With the
        # attention split by residency, tables and copies alternate on one side stream: tables
        # running ahead would let the resident parts start early and crowd the copies' compute
        # units (2.23 against 2.19 ms).
        side = self.side
        copy = side if self.split_attention else self.copy
        side.wait_stream(main)                       # fork
        if copy is not side:
            copy.wait_stream(main)
        n = sel.shape[0]
        tables, copied = [None] * hs.L, [None] * hs.L
        waits = copy_waits(hs.L)

        def resolve_tables(l):
            hs.resolve_tables(l, sel, self.slots[l], self.miss[i, l], stream=side)
            tables[l] = torch.cuda.Event()
            tables[l].record(side)

        def fetch(l):
            timing = self.fetch_events is not None
            if copy is not side and not timing:
                if l in waits:
                    copy.wait_event(tables[waits[l]])
            if copy is not side and timing and l == 0:
                copy.wait_event(tables[hs.L - 1])      # every layer's tables (one side stream)
            if timing and l == 0:
                self.fetch_events.append((torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)))
                self.fetch_events[-1][0].record(copy)
            hs.fetch_misses(l, n, stream=copy)
            if timing and l == hs.L - 1:
                self.fetch_events[-1][1].record(copy)
            copied[l] = torch.cuda.Event()
            copied[l].record(copy)

        if copy is side:
            assert self.fetch_events is None, "fetch timing needs the copies on their own stream"
            for l in range(hs.L):
                resolve_tables(l)
                fetch(l)
        else:
            for l in range(hs.L):
                resolve_tables(l)
            for l in range(hs.L):
                fetch(l)
        for l in range(hs.L):
            if self.split_attention or l >= hs.L - self.split_last:
                main.wait_event(tables[l])
                hs.attend_resident(l, q[l], self.slots[l], scale, stream=main)
                main.wait_event(copied[l])
                hs.attend_fetched(l, q[l], scale, self.out[l], self.lse[l], stream=main)
            else:
                main.wait_event(copied[l])
                if self.attend:
                    hs.attend(l, q[l], self.slots[l], scale, self.out[l], self.lse[l], stream=main)
        main.wait_stream(side)                       # join
        if copy is not side:
            main.wait_stream(copy)

    def replay(self):
        """Runs the captured steps on this object's stream (ordered after the caller's stream)."""
        dev = self.slots.device
        self.stream.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(self.stream):
            self.graph.replay()
        torch.cuda.current_stream(dev).wait_stream(self.stream)
