"""Pins of the append oracle (CPU only): hand-derived fixture, closed form
from forward-simulated histories, the allocator-independent K/V check,
untouched slots, in-place == out-of-place, inactive requests."""
import copy
import json
import os

import numpy as np
import pytest

from generative_recommendation_beam_amd.inputs import make_workload
from oracle import append as oapp
import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _run(w, inplace=True, sentinel=-7.0):
    kpool = np.full((w.num_slots, w.Hkv, w.D), sentinel)
    vpool = np.full_like(kpool, sentinel)
    table = np.full((w.N_b, w.T_max), -1, dtype=np.int64)
    ulen = np.zeros(w.R, dtype=np.int64)
    snaps = []
    for t in range(w.T_steps):
        tin = table
        tout = table if inplace else np.full_like(table, -1)
        if not inplace:
            tout[:] = table                       # ping-pong starts from the previous state
        oapp.cache_append(B=w.B, k_new=w.k_new[t].astype(np.float64),
                          v_new=w.v_new[t].astype(np.float64), parent=w.parents[t],
                          slot_base=w.slot_base, active=w.active(t), k_pool=kpool,
                          v_pool=vpool, table_in=tin, table_out=tout, unshared_len=ulen)
        table = tout
        snaps.append(table.copy())
    return kpool, vpool, table, ulen, snaps


def test_golden_lineage_table():
    g = json.load(open(os.path.join(GOLDEN, "lineage_table.json")))
    B = g["B"]
    table = np.full((B, 3), -1, dtype=np.int64)
    kpool = np.zeros((9, 1, 1))
    vpool = np.zeros_like(kpool)
    ulen = np.zeros(1, dtype=np.int64)
    for t in range(3):
        oapp.cache_append(B=B, k_new=np.zeros((B, 1, 1)), v_new=np.zeros((B, 1, 1)),
                          parent=np.array(g["parents"][t]), slot_base=np.array([g["slot_base"]]),
                          active=None, k_pool=kpool, v_pool=vpool, table_in=table,
                          table_out=table, unshared_len=ulen)
        exp = g["expect_table_after_each_step"][t]
        for b in range(B):
            assert list(table[b, :t + 1]) == exp[b]


@pytest.mark.parametrize("parent", ["uniform", "zipf", "identity"])
def test_append_closed_form_and_allocator_free(parent):
    w = make_workload("ap", R=3, B=4, Hq=2, Hkv=2, D=4, prefix_len=1, unshared_len=[5, 2, 0],
                      dtype="f32", seed_key=(200, 0), parent_dist=parent, T_max=6)
    kpool, vpool, table, ulen, _ = _run(w)
    assert list(ulen) == [5, 2, 0]
    used = set()
    for r in range(w.R):
        L = int(w.unshared_len[r])
        hist = brute.histories(w.parents, r, w.B, L)
        for b in range(w.B):
            n = r * w.B + b
            for t, a in hist[b] if L else []:
                assert table[n, t] == w.slot_base[r] + t * w.B + a   # closed form
                # allocator-independent: the referenced slot holds that step's K/V of beam a
                assert np.array_equal(kpool[table[n, t]], w.k_new[t, r * w.B + a])
                assert np.array_equal(vpool[table[n, t]], w.v_new[t, r * w.B + a])
            assert np.all(table[n, L:] == -1)                        # nothing beyond L written
            for t in range(L):
                used.add(int(w.slot_base[r]) + t * w.B + b)
    untouched = np.array(sorted(set(range(w.num_slots)) - used), dtype=np.int64)
    assert np.all(kpool[untouched] == -7.0) and np.all(vpool[untouched] == -7.0)


def test_append_inplace_equals_pingpong():
    for parent in ("uniform", "zipf"):
        w = make_workload("ip", R=2, B=7, Hq=1, Hkv=1, D=2, prefix_len=1, unshared_len=[6, 4],
                          dtype="f32", seed_key=(201, 0), parent_dist=parent)
        # adversarial patterns: all-zero, reversed, a cycle
        for pat in ("data", "zero", "reverse", "cycle"):
            w2 = copy.deepcopy(w)
            if pat != "data":
                for t in range(1, w.T_steps):
                    for r in range(w.R):
                        bb = np.arange(w.B)
                        p = {"zero": 0 * bb, "reverse": bb[::-1], "cycle": (bb + 1) % w.B}[pat]
                        w2.parents[t, r * w.B:(r + 1) * w.B] = p
            a = _run(w2, inplace=True)
            b = _run(w2, inplace=False)
            for x, y in zip(a[:4], b[:4]):
                assert np.array_equal(x, y)


def test_append_full_row_raises():
    w = make_workload("full", R=1, B=2, Hq=1, Hkv=1, D=2, prefix_len=1, unshared_len=2,
                      dtype="f32", seed_key=(202, 0), T_max=2)
    kpool, vpool, table, ulen, _ = _run(w)
    with pytest.raises(ValueError):
        oapp.cache_append(B=2, k_new=np.zeros((2, 1, 2)), v_new=np.zeros((2, 1, 2)),
                          parent=np.zeros(2, np.int64), slot_base=w.slot_base, active=None,
                          k_pool=kpool, v_pool=vpool, table_in=table, table_out=table,
                          unshared_len=ulen)
