"""The fp64 oracle over large inputs, spread over host threads.

Splitting work between calls changes nothing the oracle computes: every
decode row and every prefill row is independent of the others.  The oracle
library releases the GIL inside its calls (ctypes), so the calls run in
parallel.  Used by the full-size GPU parity tests and pinned on the CPU by
tests/test_oracle_threads.py against the unsplit calls.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

import oracle


def threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def prefill(q, kc, vc, bt, qsl, cl, scale, rows_per_task: int = 32) -> np.ndarray:
    """oracle.prefill over every row, split into sub-chunks run in threads.

    Rows r0..r1-1 of sequence s form a chunk of their own: a chunk whose last
    row sits where row r1-1 sits (context length = that row's position + 1)
    puts row r0 + i at the same position as the whole chunk does, so each
    sub-chunk's oracle rows are the whole chunk's rows."""
    ref = np.zeros(q.shape, np.float64)
    tasks = []
    for s in range(len(cl)):
        a0, a1, n = int(qsl[s]), int(qsl[s + 1]), int(cl[s])
        for r0 in range(a0, a1, rows_per_task):
            r1 = min(a1, r0 + rows_per_task)
            tasks.append((s, r0, r1, n - (a1 - r1)))

    def run(t):
        s, r0, r1, n_sub = t
        ref[r0:r1] = oracle.prefill(q[r0:r1], kc, vc, bt[s:s + 1], np.array([0, r1 - r0], np.int32),
                                    np.array([n_sub], np.int32), scale)
    with cf.ThreadPoolExecutor(max_workers=threads()) as ex:
        list(ex.map(run, tasks))
    return ref


def decode(q, kc, vc, bt, cl, scale, seqs_per_task: int = 4) -> np.ndarray:
    """oracle.decode over every sequence, a few sequences per thread task."""
    s_all = q.shape[0]
    out = np.zeros(q.shape, np.float64)
    q = np.ascontiguousarray(q)
    bt = np.ascontiguousarray(bt, dtype=np.int32)
    cl = np.ascontiguousarray(cl, dtype=np.int32)
    # longest sequences first, so that the last tasks are short
    order = np.argsort(-cl.astype(np.int64), kind="stable")
    tasks = [order[i:i + seqs_per_task] for i in range(0, s_all, seqs_per_task)]

    def run(idx):
        for s in idx:
            oracle.decode_rows_into(out, q, kc, vc, bt, cl, scale, int(s), int(s) + 1)
    with cf.ThreadPoolExecutor(max_workers=threads()) as ex:
        list(ex.map(run, tasks))
    return out
