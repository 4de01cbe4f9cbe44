"""Time the oracle on the host's cores: the CPU baseline beside the GPU figures.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py): bench.py's cpu_baseline
leg runs this module as a child process,

    python -m oracle.timing --config 5 --seconds 10 [--workers N]
                            [--single-core 1,2,4A --single-seconds 5]

and reads the one JSON object it prints. BLAS is pinned to one thread per
process here, before numpy is imported, and again in every worker.

What is timed is the oracle as it stands: per layer step, the append of the
last decode step's tokens (``oracle.append.cache_append``) and the decode
attention (``oracle.attention.attention``) over (request, kv head) units.
A unit covers the B beams of a request on the G query heads of one kv head,
i.e. B / H_kv beam-layer-steps; the append's time is charged in proportion
to the units done.
"""
from __future__ import annotations

import os

for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ[_v] = "1"

import argparse  # noqa: E402
import json  # noqa: E402
import sys  # noqa: E402
import time  # noqa: E402

import numpy as np  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from generative_recommendation_beam_amd import inputs  # noqa: E402
from oracle import append as oapp  # noqa: E402
from oracle import pool  # noqa: E402


def _cfg(s):
    return int(s) if s.isdigit() else s


def append_seconds(w):
    """Seconds of one oracle append of the last step's tokens (the cache
    holding every earlier step, built untimed)."""
    if w.T_steps == 0:
        return 0.0
    kpool = np.zeros((max(w.num_slots, 1), w.Hkv, w.D), dtype=w.k_new.dtype)
    vpool = np.zeros_like(kpool)
    table = np.full((w.N_b, w.T_max), -1, dtype=np.int64)
    ulen = np.zeros(w.R, dtype=np.int64)
    for t in range(w.T_steps - 1):
        oapp.cache_append(B=w.B, k_new=w.k_new[t], v_new=w.v_new[t], parent=w.parents[t],
                          slot_base=w.slot_base, active=w.active(t), k_pool=kpool, v_pool=vpool,
                          table_in=table, table_out=table, unshared_len=ulen)
    t = w.T_steps - 1
    tout = table.copy()
    t0 = time.perf_counter()
    oapp.cache_append(B=w.B, k_new=w.k_new[t], v_new=w.v_new[t], parent=w.parents[t],
                      slot_base=w.slot_base, active=w.active(t), k_pool=kpool, v_pool=vpool,
                      table_in=table, table_out=tout, unshared_len=ulen)
    return time.perf_counter() - t0


def time_oracle(cfg, workers, seconds):
    """Beam-layer-steps per second of the oracle on one layer of workload
    ``cfg`` over ``workers`` processes, bounded to about ``seconds``."""
    w = inputs.config(cfg, layer=0)
    t_app = append_seconds(w)
    units = pool.all_units(w)
    _, done, el, used = pool.run_units([w], units, workers=workers, seconds=seconds)
    frac = len(done) / len(units)
    beams = len(done) * w.B / w.Hkv
    total = el + t_app * frac
    return dict(value=beams / total, unit="beams*layer-steps/s", cores=used, kind="oracle",
                sample=(f"{len(done)} of {len(units)} (request, kv head) units of one layer step "
                        f"({beams:.0f} beam-layer-steps; append of the last step's tokens charged "
                        f"pro rata, {t_app:.3f} s per layer), fp64 numpy oracle, {used} worker "
                        f"process{'es' if used != 1 else ''} with one BLAS thread each, {total:.1f} s"))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", default="5")
    ap.add_argument("--seconds", type=float, default=10.0)
    ap.add_argument("--workers", type=int, default=0)
    ap.add_argument("--single-core", default="")
    ap.add_argument("--single-seconds", type=float, default=5.0)
    args = ap.parse_args()
    res = {"multi": time_oracle(_cfg(args.config), args.workers or pool.host_cores(), args.seconds)}
    single = {}
    for c in [c for c in args.single_core.split(",") if c]:
        single[c] = time_oracle(_cfg(c), 1, args.single_seconds)
    res["single_core"] = single
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
