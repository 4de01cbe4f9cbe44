"""Reference semantics of beam-search survivor selection.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py). It shares no code with the
HIP library.

xGR page, section 2.2 xBeam: each decode step keeps the Top-K sequences of a
large pool (every live beam times its best next tokens). The page's method
walks the pool with a global min-heap and stops a beam's walk as soon as a
candidate falls below the heap minimum, which is exact because a beam's
candidates come sorted. The result is the plain definition, which is what
this module computes: the n_out largest candidate scores.

Readings of points the page leaves open:
  * candidate score = beam score + token log-probability, added in float32
    (the precision the kernel adds in, so both sides decide the same order);
  * ties are broken by pool index b * K + k (smaller first), so the result is
    unique; -0.0 and +0.0 are equal scores;
  * output order is score descending (then pool index ascending): the new
    beam b' is the b'-th best candidate, its parent the candidate's beam;
  * scores are finite or -inf; NaN inputs are outside the contract.
"""
from __future__ import annotations

import numpy as np


def candidate_scores(beam_score: np.ndarray, logprob: np.ndarray) -> np.ndarray:
    """float32 [R][BW][K] = beam_score[r][b] + logprob[r][b][k], added in float32."""
    return (beam_score.astype(np.float32)[:, :, None] + logprob.astype(np.float32)).astype(np.float32)


def select(beam_score: np.ndarray, logprob: np.ndarray, token: np.ndarray, n_out: int):
    """Per request, the n_out best candidates by (score descending, pool index
    ascending). Returns parent [R][n_out] int32 (beam index), token
    [R][n_out] int32, score [R][n_out] float32."""
    R, BW, K = logprob.shape
    if not 0 <= n_out <= BW * K:
        raise ValueError("n_out out of range")
    scores = candidate_scores(beam_score, logprob)
    parent = np.empty((R, n_out), dtype=np.int32)
    tok = np.empty((R, n_out), dtype=np.int32)
    out = np.empty((R, n_out), dtype=np.float32)
    idx = np.arange(BW * K, dtype=np.int64)
    for r in range(R):
        s = scores[r].reshape(-1).astype(np.float64)
        order = np.lexsort((idx, -s))[:n_out]       # primary: -score ascending
        parent[r] = (order // K).astype(np.int32)
        tok[r] = token[r].reshape(-1)[order]
        out[r] = scores[r].reshape(-1)[order]
    return parent, tok, out
