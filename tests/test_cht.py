"""The native batch former (host C++ through the C ABI) against the
brute-force oracle: identical best candidates and batches on random
operation sequences (CPU only; the structure lives on the host)."""
import random

import pytest

from generative_recommendation_beam_amd import xattn
from oracle.cht import BruteCht


@pytest.fixture(scope="module")
def L():
    import os
    if not os.path.exists(xattn.LIB_PATH):
        from generative_recommendation_beam_amd import build
        build.build()
    return xattn.lib()


def _workload(rng, n, groups, prefix_blocks, bs):
    pre = [[rng.randint(0, 50) for _ in range(prefix_blocks * bs)] for _ in range(groups)]
    reqs = []
    for i in range(n):
        g = rng.randrange(groups)
        cut = rng.randint(0, len(pre[g]))
        toks = pre[g][:cut] + [rng.randint(0, 3) for _ in range(rng.randint(0, 3 * bs))]
        reqs.append(toks)
    return reqs


@pytest.mark.parametrize("seed", range(12))
def test_native_equals_brute_force(L, seed):
    rng = random.Random(seed)
    bs = rng.choice([1, 2, 4, 16])
    reqs = _workload(rng, 60, rng.randint(1, 4), rng.randint(1, 6), bs)
    c, o = xattn.Cht(bs), BruteCht(bs)
    nxt = 0
    for step in range(200):
        op = rng.random()
        if op < 0.35 and nxt < len(reqs):
            c.insert(nxt, reqs[nxt])
            o.insert(nxt, reqs[nxt])
            nxt += 1
        elif op < 0.6 and o.waiting:
            r, m = o.best()
            assert c.best() == (r, m)
            if rng.random() < 0.5:
                r = rng.choice(sorted(o.waiting))
            c.admit(r)
            o.admit(r)
        elif op < 0.8 and o.active:
            r = rng.choice(sorted(o.active))
            c.complete(r)
            o.complete(r)
        else:
            mb, mm = rng.randint(0, 8), rng.randint(0, 6)
            assert c.form_batch(mb, mm) == o.form_batch(mb, mm)
        assert c.best() == o.best()
    c.close()


def test_argument_errors(L):
    c = xattn.Cht(4)
    c.insert(1, [1, 2, 3, 4])
    with pytest.raises(xattn.XattnError):
        c.insert(1, [5])             # duplicate id
    with pytest.raises(xattn.XattnError):
        c.complete(1)                # not active
    c.admit(1)
    with pytest.raises(xattn.XattnError):
        c.admit(1)                   # not waiting
    c.complete(1)
    assert c.best() == (-1, -1)
    c.close()


def test_forms_homogeneous_batches_from_shuffled_groups(L):
    """The page's sensitivity experiment shape (800 requests, 8 prefix groups,
    shuffled arrival): with room for 100 and the unique tail as the missing
    budget, every formed batch is one prefix group."""
    rng = random.Random(3)
    bs, pre_blocks, tail_blocks = 16, 8, 2
    groups = [[rng.randint(0, 30000) for _ in range(pre_blocks * bs)] for _ in range(8)]
    order = [g for g in range(8) for _ in range(100)]
    rng.shuffle(order)
    c = xattn.Cht(bs)
    for rid, g in enumerate(order):
        c.insert(rid, groups[g] + [rng.randint(0, 30000) for _ in range(tail_blocks * bs)])
    seen = 0
    while True:
        batch = c.form_batch(100, tail_blocks)
        if not batch:
            break
        assert len(batch) == 100 and len({order[r] for r in batch}) == 1
        for r in batch:
            c.complete(r)
        seen += len(batch)
    assert seen == 800
    c.close()
