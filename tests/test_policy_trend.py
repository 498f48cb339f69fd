"""The miss-count trend the HiSparse note reports (section 3, Fig. 3): a larger device buffer
gives fewer misses, and LRU gives fewer than policies that do not exploit locality.  A soft
check, not an invariant (batched steps with ties do not guarantee LRU inclusion), run on the
oracle over a reduced copy of the buffer-sweep workload with fixed seeds."""
import numpy as np

import oracle
from synth import configs as C
from synth import trace as tr


def test_bigger_buffer_and_lru_give_fewer_misses():
    w0 = C.SWEEP.with_(n=6, steps=50)
    trace = tr.generate(w0.trace_spec(), steps=w0.steps)
    steady = {}
    for B in C.SWEEP_BUFFERS:
        w = C.sweep_point(B).with_(n=6)
        for pol in (oracle.LRU, oracle.FIFO, oracle.RANDOM):
            oc = oracle.OracleCache(w.n, 1, B, w.cap, policy=pol, seed=12345)
            m = [oc.resolve(0, trace[t])[1].mean() for t in range(w0.steps)]
            steady[B, pol] = float(np.mean(m[10:]))
    for pol in (oracle.LRU, oracle.FIFO, oracle.RANDOM):
        assert steady[2048, pol] > steady[4096, pol] > steady[6144, pol]
    # with B = k every policy must hold exactly the selection: no choice, equal misses
    assert steady[2048, oracle.LRU] == steady[2048, oracle.FIFO] == steady[2048, oracle.RANDOM]
    for B in (4096, 6144):
        assert steady[B, oracle.LRU] < min(steady[B, oracle.FIFO], steady[B, oracle.RANDOM])
