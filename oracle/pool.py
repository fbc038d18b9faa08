"""Row-parallel evaluation of the oracle on a pool of worker processes.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: used by ``tests/`` and by the
``cpu_baseline`` leg of ``bench.py``.  It adds no arithmetic: every output row is the one
``paged_attention`` / ``sparse_attention`` compute for it (their ``rows`` argument), the
rows are only dealt out to processes and put back in order, and the status words are
OR-ed.  Workers are started with the "spawn" method (they import numpy and this package
only, never the GPU library) and each runs its BLAS on one thread.
"""
from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

_STATE = {}


def default_workers(cap: int = 16) -> int:
    """Cores this process may run on (its CPU affinity), at most ``cap``."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def _init(fn_name, args, kwargs):
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)
    from . import attention
    _STATE["fn"] = getattr(attention, fn_name)
    _STATE["args"] = args
    _STATE["kwargs"] = kwargs


def _run(rows):
    out, status = _STATE["fn"](*_STATE["args"], **_STATE["kwargs"], rows=rows)
    return out, status


def map_rows(fn_name: str, args: tuple, kwargs: dict, rows, workers: int, chunk: int = 64):
    """``oracle.<fn_name>(*args, **kwargs, rows=rows)`` evaluated over ``workers``
    processes, ``chunk`` rows per task.  ``rows`` must be increasing (the oracle returns
    rows in increasing order).  Returns ``(out, status)`` as the single call would."""
    rows = [int(r) for r in rows]
    assert all(a < b for a, b in zip(rows, rows[1:])), "rows must be increasing"
    tasks = [rows[i:i + chunk] for i in range(0, len(rows), chunk)]
    if workers <= 1 or len(tasks) <= 1:
        from . import attention
        return getattr(attention, fn_name)(*args, **kwargs, rows=rows)
    ctx = mp.get_context("spawn")
    with ProcessPoolExecutor(max_workers=min(workers, len(tasks)), mp_context=ctx,
                             initializer=_init, initargs=(fn_name, args, kwargs)) as ex:
        parts = list(ex.map(_run, tasks))
    status = 0
    for _, st in parts:
        status |= st
    return np.concatenate([o for o, _ in parts], axis=0), status
