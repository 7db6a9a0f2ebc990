"""Row-chunked, thread-parallel calls of the CPU oracle for the full-size
parity tests.

The oracle quantizes rows independently, so the full-size layers are cut
into chunks of rows that run on a thread pool (numpy releases the GIL inside
its array operations).  Nothing here computes anything itself: every code,
scale byte and product comes from the oracle's own functions.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle

CHUNK = 128


def threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _chunks(n):
    return [(r0, min(n, r0 + CHUNK)) for r0 in range(0, n, CHUNK)]


def quant_act(x, s, offsets=None):
    """oracle.quant_act over all rows of x, in row chunks.  x: [M, K] bf16
    bits or fp32; s: [E, K]; offsets: [E+1] or None."""
    M = x.shape[0]
    off = None if offsets is None else np.asarray(offsets, dtype=np.int64)

    def one(rr):
        r0, r1 = rr
        o = None if off is None else np.clip(off - r0, 0, r1 - r0)
        return oracle.quant_act(x[r0:r1], s, o)

    with ThreadPoolExecutor(threads()) as ex:
        parts = list(ex.map(one, _chunks(M)))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def prepare_weights(w, s):
    """oracle.prepare_weights of one expert's [N, K] weights, in row chunks."""
    N = w.shape[0]
    with ThreadPoolExecutor(threads()) as ex:
        parts = list(ex.map(lambda rr: oracle.prepare_weights(w[rr[0]:rr[1]], s), _chunks(N)))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])
