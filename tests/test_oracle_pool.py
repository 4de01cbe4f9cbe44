"""Pins of the oracle's process-pool driver (CPU only).

``oracle.pool`` only distributes (request, kv head) units of
``oracle.attention.attention`` over worker processes and reassembles their
output slices; these tests check that the assembled result is exactly the
plain function's, bit for bit, on ragged workloads (a wrong slice, a missing
or duplicated unit, or a unit that computes too much would all show), and
that the time-bounded runner reports exactly the units it finished.
"""
import numpy as np
import pytest

from generative_recommendation_beam_amd.inputs import make_workload
from oracle import attention as oa
from oracle import pool


def ragged(seed=5):
    return make_workload("pool", R=3, B=5, Hq=8, Hkv=2, D=16, prefix_len=[37, 0, 70],
                         unshared_len=[2, 3, 0], dtype="bf16", seed_key=(210, seed),
                         parent_dist="uniform")


@pytest.mark.parametrize("workers", [1, 3])
def test_parallel_equals_plain_bitwise(workers):
    w = ragged()
    O, L = oa.attention(w)
    Op, Lp, dt, used = pool.attention_parallel(w, workers=workers)
    assert used == workers
    assert not np.isnan(Op).any() and not np.isnan(Lp).any()
    assert np.array_equal(Op, O)
    # lse of an empty request is -inf on both sides; every other entry equal
    assert np.array_equal(np.isneginf(Lp), np.isneginf(L))
    fin = np.isfinite(L)
    assert np.array_equal(Lp[fin], L[fin])


def test_subset_of_units_fills_only_those():
    w = ragged(6)
    O, L = oa.attention(w)
    units = [(2, 1), (0, 0)]
    Op, Lp, _, _ = pool.attention_parallel(w, units=units, workers=2)
    G = w.Hq // w.Hkv
    mask = np.zeros((w.N_b, w.Hq), dtype=bool)
    for r, h in units:
        mask[r * w.B:(r + 1) * w.B, h * G:(h + 1) * G] = True
    assert np.array_equal(Op[mask], O[mask])
    assert np.isnan(Op[~mask]).all() and np.isnan(Lp[~mask]).all()


def test_time_bounded_run_counts_what_it_finished():
    w = ragged(7)
    units = pool.all_units(w)
    outs, done, el, used = pool.run_units([w], units, workers=2, seconds=0.0)
    assert 1 <= len(done) <= len(units)
    assert len(set(done)) == len(done)
    O, L = oa.attention(w)
    G = w.Hq // w.Hkv
    for _, r, h in done:
        sl = (slice(r * w.B, (r + 1) * w.B), slice(h * G, (h + 1) * G))
        assert np.array_equal(outs[0][0][sl], O[sl])
    finished = {(r, h) for _, r, h in done}
    for r in range(w.R):
        for h in range(w.Hkv):
            if (r, h) not in finished:
                assert np.isnan(outs[0][0][r * w.B:(r + 1) * w.B, h * G:(h + 1) * G]).all()


def test_workers_pin_blas_to_one_thread():
    from threadpoolctl import threadpool_info
    lim = pool._pin_blas()
    try:
        assert all(i.get("num_threads", 1) == 1 for i in threadpool_info())
    finally:
        lim.restore_original_limits()


def test_timing_child_reports_a_bounded_sample():
    """oracle.timing, the child process bench.py runs, pins BLAS through the
    environment before numpy loads and prints one JSON object."""
    import json
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-m", "oracle.timing", "--config", "1", "--seconds", "1",
                          "--workers", "2", "--single-core", "1", "--single-seconds", "1"],
                         cwd=root, capture_output=True, text=True, timeout=120, check=True)
    res = json.loads(out.stdout.strip().splitlines()[-1])
    m = res["multi"]
    assert m["kind"] == "oracle" and m["unit"] == "beams*layer-steps/s" and m["value"] > 0
    assert m["cores"] == 1  # config 1 has a single (request, kv head) unit
    assert res["single_core"]["1"]["cores"] == 1
