"""Oracle scores of whole KV heads at full size, computed in worker processes.

Test infrastructure: the only arithmetic here is oracle.waits_oracle's.  A
KV head's score is a sum over its query heads g and the query rows q of the
prompt (WAITS README, introduction), so it splits into pieces over disjoint
(query head, row range) parts that add up to the whole.  Each piece is
``head_scores`` of one query head on the prompt's prefix up to the end of
the range, with the rows before the range left out (``row_min``); rows only
reach keys at or before them, so a piece is exact on every key it returns.
The pieces run in a pool of fresh interpreters (spawned, so no GPU state is
inherited) with one BLAS thread each, and are added in a fixed order.
"""
from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np


def workers() -> int:
    """Worker processes: the host cores this process may use, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:  # pragma: no cover
        pass


def _piece(args):
    from oracle import waits_oracle as orc
    qg, kh, w, scale, r0, weight_floor = args
    return orc.head_scores(qg, kh, w, scale, weight_floor=weight_floor, row_min=r0)


def _cuts(w: np.ndarray, weight_floor: float, pieces: int):
    """Row ranges [r0, r1) of about equal work (a row costs q + 1 keys)."""
    rows = np.nonzero((w != 0.0) & (w > weight_floor))[0]
    if len(rows) == 0:
        return []
    work = np.cumsum(rows + 1.0)
    bounds = [0]
    for i in range(1, pieces):
        j = int(np.searchsorted(work, work[-1] * i / pieces))
        r = int(rows[min(j, len(rows) - 1)])
        if r > bounds[-1]:
            bounds.append(r)
    bounds.append(int(rows[-1]) + 1)
    return list(zip(bounds[:-1], bounds[1:]))


def kv_head_scores(q, k, h: int, group: int, a: float, b: int, scale: float,
                   weight_floor: float = 0.0, pool=None) -> np.ndarray:
    """float64 scores [N] of KV head ``h`` of one prompt (q [N, Hq, d],
    k [N, Hkv, d] float32 values), the sum over its ``group`` query heads."""
    from oracle import waits_oracle as orc
    n = q.shape[0]
    w = orc.sigmoid_weights(n, a, b)
    scale64 = float(np.float32(scale))
    nw = workers()
    per_head = max(1, (2 * nw + group - 1) // group)
    tasks, spans = [], []
    for j in range(group):
        g = h * group + j
        for r0, r1 in _cuts(w, weight_floor, per_head):
            qg = np.ascontiguousarray(q[None, :r1, g])
            kh = np.ascontiguousarray(k[:r1, h])
            tasks.append((qg, kh, w[:r1], scale64, r0, weight_floor))
            spans.append(r1)
    s = np.zeros(n, dtype=np.float64)
    own = pool is None
    if own:
        pool = ProcessPoolExecutor(nw, mp_context=mp.get_context("spawn"), initializer=_init)
    try:
        for r1, part in zip(spans, pool.map(_piece, tasks)):
            s[:r1] += part
    finally:
        if own:
            pool.shutdown()
    return s


def make_pool() -> ProcessPoolExecutor:
    """A pool to share across several kv_head_scores calls."""
    return ProcessPoolExecutor(workers(), mp_context=mp.get_context("spawn"), initializer=_init)
