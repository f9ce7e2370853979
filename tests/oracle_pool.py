"""Expert FFNs of the fp64 oracle evaluated in worker processes, for checks
over many experts of the full-size layers (each expert's dequantisation takes
about a second of one core).  The workers import only NumPy and the oracle;
they receive each expert's packed bytes and activation rows and run
oracle.expert_ffn on them."""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

import oracle

_POOL = None


def _init():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)


def _task(args):
    wfmt, gate, up, down, X = args
    src = oracle.ExpertSource(wfmt, gate, up, down)
    return oracle.expert_ffn(src, 0, X)


def pool():
    global _POOL
    if _POOL is None:
        n = max(1, min(16, os.cpu_count() or 1))
        _POOL = mp.get_context("spawn").Pool(n, initializer=_init)
    return _POOL


def packed(src, e):
    """(gate, up, down) of expert e of `src` as host arrays with a leading
    expert dimension of one, in the layout oracle.ExpertSource takes."""
    if isinstance(src, oracle.ExpertSource):
        return tuple(tuple(None if a is None else a[e:e + 1] for a in getattr(src, p))
                     for p in ("gate", "up", "down"))
    return src.packed(e)


def expert_ffns(jobs, chunk=24):
    """jobs: list of (source, expert, X rows float64) -> list of FFN outputs,
    in order.  Packed bytes are fetched `chunk` experts at a time."""
    out = []
    for i in range(0, len(jobs), chunk):
        part = jobs[i:i + chunk]
        tasks = [(src.wfmt, *packed(src, e), np.ascontiguousarray(X)) for src, e, X in part]
        out.extend(pool().map(_task, tasks, chunksize=1))
    return out
