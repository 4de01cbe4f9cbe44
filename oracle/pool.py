"""Run the oracle over many host cores (used to time it as a CPU baseline).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py). The arithmetic is exactly
``oracle.attention.attention``; this module only hands (request, kv head)
units to forked worker processes, each limited to one BLAS thread, and
gathers their outputs.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import time

import numpy as np

from . import attention as _att

_W = None


def _init_worker():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover - threadpoolctl missing
        pass


def _unit(args):
    r, h = args
    o, lse = _att.attention(_W, requests=[r], heads=[h])
    G = _W.Hq // _W.Hkv
    sl = slice(r * _W.B, (r + 1) * _W.B)
    return r, h, o[sl, h * G:(h + 1) * G], lse[sl, h * G:(h + 1) * G]


def host_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def attention_parallel(w, units=None, workers=None):
    """Oracle attention over the given (r, h) units on ``workers`` processes.

    Returns (O, lse, seconds, workers) with O / lse NaN outside the units.
    """
    global _W
    if units is None:
        units = [(r, h) for r in range(w.R) for h in range(w.Hkv)]
    workers = workers or host_cores()
    workers = max(1, min(workers, len(units)))
    O = np.full((w.N_b, w.Hq, w.D), np.nan)
    LSE = np.full((w.N_b, w.Hq), np.nan)
    G = w.Hq // w.Hkv
    _W = w
    t0 = time.perf_counter()
    if workers == 1:
        _init_worker()
        results = map(_unit, units)
        for r, h, o, lse in results:
            O[r * w.B:(r + 1) * w.B, h * G:(h + 1) * G] = o
            LSE[r * w.B:(r + 1) * w.B, h * G:(h + 1) * G] = lse
    else:
        ctx = mp.get_context("fork")
        with ctx.Pool(workers, initializer=_init_worker) as pool:
            for r, h, o, lse in pool.imap_unordered(_unit, units):
                O[r * w.B:(r + 1) * w.B, h * G:(h + 1) * G] = o
                LSE[r * w.B:(r + 1) * w.B, h * G:(h + 1) * G] = lse
    dt = time.perf_counter() - t0
    _W = None
    return O, LSE, dt, workers
