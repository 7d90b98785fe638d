"""Whole-workload oracle results for the GPU parity tests.

The oracle works on one (batch, head) at a time. Here it is called on every
(batch, head) slice of a workload, in a pool of threads (NumPy releases the
interpreter lock inside its large array operations and BLAS calls, so heads
run in parallel; BLAS itself is held to one thread per call), and the
per-head results are put back into whole tensors. Nothing here computes
attention: each slice's result is exactly what the oracle function returns
for it.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
from threadpoolctl import threadpool_limits


def workers() -> int:
    """Threads for the oracle: the CPUs this process may run on, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def head(x, b, h):
    """The [1, N, 1, d] slice of a [B, N, H, d] array for (batch b, head h)."""
    return x[b : b + 1, :, h : h + 1, :]


def by_head(fn, B, H, layouts):
    """Call fn(b, h) for every (batch, head) and assemble its outputs.

    fn returns a tuple whose i-th entry is laid out as layouts[i]: "bnhd"
    ([1, N, 1, d] -> a [B, N, H, d] array) or "bhn" ([1, 1, N] -> [B, H, N]).
    Entries past len(layouts) are dropped."""
    pairs = [(b, h) for b in range(B) for h in range(H)]
    with threadpool_limits(1), ThreadPoolExecutor(workers()) as ex:
        res = list(ex.map(lambda bh: fn(*bh)[: len(layouts)], pairs))
    outs = []
    for i, lay in enumerate(layouts):
        first = np.asarray(res[0][i])
        if lay == "bnhd":
            full = np.empty((B, first.shape[1], H, first.shape[3]))
            for (b, h), r in zip(pairs, res):
                full[b, :, h, :] = r[i][0, :, 0, :]
        elif lay == "bhn":
            full = np.empty((B, H, first.shape[2]))
            for (b, h), r in zip(pairs, res):
                full[b, h, :] = r[i][0, 0, :]
        else:
            raise ValueError(f"unknown layout {lay}")
        outs.append(full)
    return outs
