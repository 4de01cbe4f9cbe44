"""Pins of the beam-search selection oracle (CPU only).

The oracle is a full sort. It is checked against (1) a brute-force repeated
maximum written out in plain Python, (2) the page's own method, a global
min-heap walk that stops a beam's candidates early (xGR page, section 2.2
xBeam), written independently with heapq, and (3) properties any correct
selection has, on larger inputs of every distribution.
"""
import heapq
import math

import numpy as np
import pytest

from generative_recommendation_beam_amd.inputs import make_topk
from oracle import beam_topk as bt


def _brute(beam_score, logprob, token, n_out):
    R, BW, K = logprob.shape
    res = []
    for r in range(R):
        cands = []
        for b in range(BW):
            for k in range(K):
                s = float(np.float32(np.float32(beam_score[r, b]) + np.float32(logprob[r, b, k])))
                cands.append((s, b * K + k))
        chosen = []
        taken = set()
        for _ in range(n_out):
            best = None
            for s, i in cands:
                if i in taken:
                    continue
                if best is None or s > best[0] or (s == best[0] and i < best[1]):
                    best = (s, i)
            taken.add(best[1])
            chosen.append(best)
        res.append([(i // K, int(token[r, i // K, i % K]), s) for s, i in chosen])
    return res


def _heap_walk(beam_score, logprob, token, n_out):
    """Global min-heap of the best n_out so far; a beam's walk stops at the
    first candidate that cannot enter the heap (its later ones are smaller)."""
    R, BW, K = logprob.shape
    res = []
    for r in range(R):
        heap = []  # (score, -index): the heap minimum is the worst kept candidate
        visited = 0
        for b in range(BW):
            for k in range(K):
                s = float(np.float32(np.float32(beam_score[r, b]) + np.float32(logprob[r, b, k])))
                item = (s, -(b * K + k))
                visited += 1
                if len(heap) < n_out:
                    heapq.heappush(heap, item)
                elif item > heap[0]:
                    heapq.heapreplace(heap, item)
                else:
                    break  # early termination for this beam
        best = sorted(heap, reverse=True)
        res.append(([(-i // K, int(token[r, -i // K, -i % K]), s) for s, i in best], visited))
    return res


def _as_lists(parent, tok, score):
    return [[(int(parent[r, i]), int(tok[r, i]), float(score[r, i])) for i in range(parent.shape[1])]
            for r in range(parent.shape[0])]


@pytest.mark.parametrize("dist", ["softmax", "ties", "masked", "equal"])
@pytest.mark.parametrize("BW,K,n_out", [(4, 3, 4), (5, 4, 3), (3, 6, 10), (6, 1, 6), (4, 4, 16)])
def test_oracle_equals_brute_force(dist, BW, K, n_out):
    x = make_topk("tiny", R=2, BW=BW, K=K, n_out=n_out, seed_key=(1, BW, K), dist=dist, vocab=32)
    got = _as_lists(*bt.select(x.beam_score, x.logprob, x.token, x.n_out))
    assert got == _brute(x.beam_score, x.logprob, x.token, x.n_out)


@pytest.mark.parametrize("dist", ["softmax", "ties", "masked", "equal"])
@pytest.mark.parametrize("BW,K", [(32, 32), (64, 16), (16, 64)])
def test_oracle_equals_heap_walk_with_early_termination(dist, BW, K):
    x = make_topk("walk", R=2, BW=BW, K=K, seed_key=(2, BW, K), dist=dist, vocab=512)
    got = _as_lists(*bt.select(x.beam_score, x.logprob, x.token, x.n_out))
    walk = _heap_walk(x.beam_score, x.logprob, x.token, x.n_out)
    assert got == [w for w, _ in walk]
    if dist == "softmax":  # the early stop skips most of the pool
        assert all(v < 0.5 * BW * K for _, v in walk)


@pytest.mark.parametrize("dist", ["softmax", "ties", "masked"])
def test_oracle_properties(dist):
    x = make_topk("prop", R=3, BW=128, K=128, seed_key=(3, 0), dist=dist)
    parent, tok, score = bt.select(x.beam_score, x.logprob, x.token, x.n_out)
    s_all = bt.candidate_scores(x.beam_score, x.logprob)
    for r in range(x.R):
        sel = [(float(score[r, i]), int(parent[r, i])) for i in range(x.n_out)]
        # sorted by score descending
        assert all(sel[i][0] >= sel[i + 1][0] for i in range(len(sel) - 1))
        # each output matches its input candidate
        kk = [int(np.nonzero(x.token[r, p] == t)[0][0]) for (_, p), t in zip(sel, tok[r])]
        for (s, p), k in zip(sel, kk):
            assert np.float32(s) == s_all[r, p, k]
        # nothing left out beats the worst kept one
        chosen = {int(p) * x.K + k for (_, p), k in zip(sel, kk)}
        worst = min((s, -(p * x.K + k)) for (s, p), k in zip(sel, kk))
        flat = s_all[r].reshape(-1)
        for i in range(flat.size):
            if i not in chosen:
                assert (float(flat[i]), -i) < worst


def test_oracle_special_cases():
    # one candidate per beam: the beams themselves, re-sorted by score
    x = make_topk("k1", R=1, BW=50, K=1, seed_key=(4, 0))
    parent, tok, score = bt.select(x.beam_score, x.logprob, x.token, 50)
    expect = sorted(range(50), key=lambda b: (-float(np.float32(x.beam_score[0, b] + x.logprob[0, b, 0])), b))
    assert list(parent[0]) == expect
    # all equal: the first n_out pool indices, in order
    x = make_topk("eq", R=1, BW=7, K=5, n_out=12, seed_key=(4, 1), dist="equal")
    parent, tok, score = bt.select(x.beam_score, x.logprob, x.token, 12)
    assert list(parent[0] * 5 + tok[0]) == list(range(12))
    # n_out = whole pool: a full sort
    x = make_topk("all", R=1, BW=6, K=4, n_out=24, seed_key=(4, 2))
    parent, tok, score = bt.select(x.beam_score, x.logprob, x.token, 24)
    assert sorted(zip(parent[0], tok[0])) == sorted((b, int(x.token[0, b, k])) for b in range(6) for k in range(4))
    # -0.0 and +0.0 tie; the smaller index wins
    bs = np.array([[0.0, -0.0]], np.float32)
    lp = np.array([[[-0.0], [0.0]]], np.float32)
    parent, tok, score = bt.select(bs, lp, np.zeros((1, 2, 1), np.int32), 2)
    assert list(parent[0]) == [0, 1]
    # -inf candidates come last, by index
    lp = np.array([[[-1.0, -math.inf], [-math.inf, -math.inf]]], np.float32)
    bs = np.zeros((1, 2), np.float32)
    parent, tok, score = bt.select(bs, lp, np.arange(4, dtype=np.int32).reshape(1, 2, 2), 4)
    assert list(tok[0]) == [0, 1, 2, 3]


def test_inputs_rows_sorted():
    for dist in ("softmax", "ties", "masked", "equal"):
        x = make_topk("s", R=2, BW=16, K=32, seed_key=(5, 0), dist=dist)
        assert np.all(x.logprob[:, :, :-1] >= x.logprob[:, :, 1:])
        assert np.all(x.beam_score[:, :-1] >= x.beam_score[:, 1:])
