"""Row-parallel evaluation of the oracle on a pool of worker processes.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: used by ``tests/`` and by the
``cpu_baseline`` leg of ``bench.py``.  It adds no arithmetic: every output row is the one
``paged_attention`` / ``sparse_attention`` compute for it (their ``rows`` argument), the
rows are only dealt out to processes and put back in order, and the status words are
OR-ed.  Workers import numpy and this package only (never the GPU library), and each runs
its BLAS on one thread.  ``map_rows`` starts them with the "spawn" method, which is safe in
a process that already uses the GPU; ``run_for`` (the timed CPU baseline) may "fork"
them, sharing the parent's arrays without copies, when the GPU has not been initialised.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import time
from concurrent.futures import FIRST_COMPLETED, ProcessPoolExecutor, wait

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


def run_for(fn_name: str, args: tuple, kwargs: dict, rows, workers: int, seconds: float,
            chunk: int = 8, method: str = "spawn"):
    """Evaluate ``oracle.<fn_name>`` on chunks of ``rows`` (cycling through them) on
    ``workers`` processes, keeping every worker busy, until ``seconds`` of wall time have
    passed.  Returns ``(rows_done, elapsed_s)``: the row ids of every completed chunk (with
    repeats) and the time from the first submission to the last completion, worker start-up
    excluded."""
    rows = [int(r) for r in rows]
    chunks = [rows[i:i + chunk] for i in range(0, len(rows), chunk)]
    ctx = mp.get_context(method)
    done = []
    with ProcessPoolExecutor(max_workers=workers, mp_context=ctx, initializer=_init,
                             initargs=(fn_name, args, kwargs)) as ex:
        # start every worker (imports, initializer) before the clock starts
        list(ex.map(_ready, range(4 * workers)))
        nxt = 0
        pending = set()
        t0 = time.perf_counter()
        for _ in range(2 * workers):
            pending.add(ex.submit(_tagged, chunks[nxt % len(chunks)]))
            nxt += 1
        t_end = t0
        while pending:
            fin, pending = wait(pending, return_when=FIRST_COMPLETED)
            for f in fin:
                done.extend(f.result())
                t_end = time.perf_counter()
                if t_end - t0 < seconds:
                    pending.add(ex.submit(_tagged, chunks[nxt % len(chunks)]))
                    nxt += 1
    return done, t_end - t0


def _ready(_):
    return os.getpid()


def _tagged(rows):
    _run(rows)
    return rows
