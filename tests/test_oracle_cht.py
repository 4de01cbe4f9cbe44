"""Pins of the brute-force batch-forming oracle (CPU): hand-worked cases and
properties that any correct missing count has."""
import random

from oracle.cht import BruteCht


def test_hand_worked_missing_counts_and_best():
    c = BruteCht(2)
    c.insert(10, [1, 2, 3, 4, 5, 6])   # blocks (1,2)(3,4)(5,6)
    c.insert(11, [1, 2, 3, 4, 9, 9])   # shares 2 blocks with 10
    c.insert(12, [1, 2, 7, 7])         # shares 1 block with 10 and 11
    c.insert(13, [8, 8, 8, 8, 8])      # 2 full blocks, shares none; the 5th token is a partial block
    c.insert(14, [1, 2, 3])            # 1 full block
    # nothing active: missing = full blocks; best is the fewest, then the earliest
    assert [c.missing(r) for r in (10, 11, 12, 13, 14)] == [3, 3, 2, 2, 1]
    assert c.best() == (14, 1)
    c.admit(10)
    assert [c.missing(r) for r in (11, 12, 13, 14)] == [1, 1, 2, 0]
    assert c.best() == (14, 0)
    c.admit(14)
    assert c.best() == (11, 1)         # ties with 12 at 1; 11 came first
    c.admit(11)
    assert c.missing(12) == 1 and c.missing(13) == 2
    c.complete(10)
    c.complete(11)                     # active: {14} = (1,2)
    assert c.missing(12) == 1 and c.missing(13) == 2
    c.complete(14)                     # nothing active
    assert c.missing(12) == 2


def test_form_batch_groups_a_shared_prefix():
    c = BruteCht(4)
    pre = [[g * 100 + i for i in range(16)] for g in range(3)]  # 4 blocks each
    rid = 0
    for k in range(4):
        for g in range(3):
            c.insert(rid, pre[g] + [1000 + rid] * 8)  # 2 private blocks each
            rid += 1
    batch = c.form_batch(max_batch=8, max_missing=2)
    # seeded with request 0 (group 0); then its 3 group-mates (missing 2 each)
    assert batch == [0, 3, 6, 9]
    assert c.best()[1] == 6


def test_properties_random():
    rng = random.Random(7)
    for trial in range(20):
        c = BruteCht(rng.choice([1, 2, 4]))
        live = []
        for rid in range(30):
            base = rng.choice([[1, 2, 3, 4, 5, 6, 7, 8], [1, 2, 3, 4, 9, 9, 9, 9], [5, 5, 5, 5]])
            toks = base[:rng.randint(0, len(base))] + [rng.randint(0, 3) for _ in range(rng.randint(0, 9))]
            c.insert(rid, toks)
            live.append(rid)
        for step in range(40):
            w = sorted(c.waiting)
            if not w:
                break
            before = {r: c.missing(r) for r in w}
            for r in w:
                assert 0 <= before[r] <= c.nblocks(r)
            r = rng.choice(w)
            c.admit(r)
            for x in c.waiting:   # admitting can only cover more blocks
                assert c.missing(x) <= before[x]
            # a waiting request identical to an active one misses nothing
            for x in c.waiting:
                if any(c.tokens[x][:c.nblocks(x) * c.bs] == c.tokens[a][:c.nblocks(x) * c.bs] and
                       c.nblocks(a) >= c.nblocks(x) for a in c.active):
                    assert c.missing(x) == 0
            if c.active and rng.random() < 0.3:
                c.complete(rng.choice(sorted(c.active)))
