"""Run the oracle over many host cores (used to time it as a CPU baseline).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py). The arithmetic is exactly
``oracle.attention.attention``; this module only hands (workload, request,
kv head) units to forked worker processes and puts their output slices back
in place. ``tests/test_oracle_pool.py`` pins it: on ragged workloads its
assembled outputs equal ``attention`` bit for bit, with one worker and with
several.

BLAS threads: every worker limits its BLAS library to one thread and checks
that the limit took (a worker whose BLAS still reports more threads raises).
The timing entry point (``oracle/timing.py``) also sets OMP_NUM_THREADS,
OPENBLAS_NUM_THREADS and MKL_NUM_THREADS to 1 before numpy is imported, so
its workers start pinned.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import time

import numpy as np

from . import attention as _att

_WS = None  # workloads the forked workers read (set before the pool forks)


def _pin_blas():
    """Limit this process's BLAS / OpenMP pools to one thread; raise if a
    library still reports more. Returns the limiter (whose
    ``restore_original_limits()`` undoes it)."""
    from threadpoolctl import threadpool_info, threadpool_limits
    lim = threadpool_limits(1)
    wide = [i for i in threadpool_info() if i.get("num_threads", 1) != 1]
    if wide:
        raise RuntimeError(f"oracle worker: BLAS still multi-threaded after the limit: {wide}")
    return lim


def _unit(args):
    """Oracle attention of one (request r, kv head h) of workload i: the B
    beams x G query heads that read that kv head."""
    i, r, h = args
    w = _WS[i]
    o, lse = _att.attention(w, requests=[r], heads=[h])
    G = w.Hq // w.Hkv
    sl = slice(r * w.B, (r + 1) * w.B)
    return i, r, h, o[sl, h * G:(h + 1) * G], lse[sl, h * G:(h + 1) * G]


def host_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def all_units(w, i=0):
    return [(i, r, h) for r in range(w.R) for h in range(w.Hkv)]


def run_units(workloads, units, workers=None, seconds=None):
    """Oracle attention over ``units`` ((workload index, r, h) triples) on
    ``workers`` forked processes.

    With ``seconds``, no unit is started once that many seconds have passed
    (units already running finish and count). Returns (outs, done, elapsed,
    workers): outs[i] = (O, lse) of workload i, NaN outside the units done;
    done = the units completed.
    """
    global _WS
    workers = max(1, min(workers or host_cores(), len(units) or 1))
    outs = [(np.full((w.N_b, w.Hq, w.D), np.nan), np.full((w.N_b, w.Hq), np.nan)) for w in workloads]
    done = []

    def put(res):
        i, r, h, o, lse = res
        w = workloads[i]
        G = w.Hq // w.Hkv
        outs[i][0][r * w.B:(r + 1) * w.B, h * G:(h + 1) * G] = o
        outs[i][1][r * w.B:(r + 1) * w.B, h * G:(h + 1) * G] = lse
        done.append((i, r, h))

    _WS = list(workloads)
    t0 = time.perf_counter()
    try:
        if workers == 1:
            lim = _pin_blas()
            try:
                for u in units:
                    if seconds is not None and done and time.perf_counter() - t0 >= seconds:
                        break
                    put(_unit(u))
            finally:
                lim.restore_original_limits()
        else:
            ctx = mp.get_context("fork")
            with ctx.Pool(workers, initializer=_pin_blas) as pool:
                pending = []
                it = iter(units)
                exhausted = False
                while True:
                    while not exhausted and len(pending) < workers and (
                            seconds is None or time.perf_counter() - t0 < seconds or not (done or pending)):
                        u = next(it, None)
                        if u is None:
                            exhausted = True
                            break
                        pending.append(pool.apply_async(_unit, (u,)))
                    if not pending:
                        break
                    pending[0].wait()
                    still = []
                    for p in pending:
                        if p.ready():
                            put(p.get())
                        else:
                            still.append(p)
                    pending = still
                    if seconds is not None and time.perf_counter() - t0 >= seconds:
                        exhausted = True
        elapsed = time.perf_counter() - t0
    finally:
        _WS = None
    return outs, done, elapsed, workers


def attention_parallel(w, units=None, workers=None):
    """Oracle attention of workload w over the given (r, h) units (all by
    default) on ``workers`` processes.

    Returns (O, lse, seconds, workers) with O / lse NaN outside the units.
    """
    units = [(0, r, h) for (r, h) in units] if units is not None else all_units(w)
    outs, _, dt, used = run_units([w], units, workers)
    return outs[0][0], outs[0][1], dt, used
