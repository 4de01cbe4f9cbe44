"""Brute-force pins for the oracle: scalar Python loops over tiny inputs.

These re-derive the method from its statement rather than from the oracle's
code: a beam's history is built by simulating the decode steps FORWARD (each
new beam takes a copy of its parent's history and appends its own token),
where the oracle walks parent links backwards; scores, max, exponentials and
sums are plain loops over explicitly listed keys.
"""
from __future__ import annotations

import math

import numpy as np

from generative_recommendation_beam_amd.inputs import to_f64


def histories(parents, r, B, L):
    """hist[b] = [(t, owner beam)] for t = 0..L-1, built forward in time."""
    hist = [[] for _ in range(B)]
    for t in range(L):
        if t == 0:
            hist = [[(0, b)] for b in range(B)]
        else:
            hist = [list(hist[int(parents[t][r * B + b])]) + [(t, b)] for b in range(B)]
    return hist


def beam_keys(w, r, b, h, *, prefix=True, generated=True):
    """Explicit list of (k, v) float vectors of beam b's full key sequence."""
    ks, vs = [], []
    kS, vS = to_f64(w.k_shared), to_f64(w.v_shared)
    kN, vN = to_f64(w.k_new), to_f64(w.v_new)
    if prefix:
        off = int(w.prefix_off[r])
        for j in range(int(w.prefix_len[r])):
            ks.append(list(kS[h, off + j]))
            vs.append(list(vS[h, off + j]))
    if generated:
        for (t, a) in histories(w.parents, r, w.B, int(w.unshared_len[r]))[b]:
            ks.append(list(kN[t, r * w.B + a, h]))
            vs.append(list(vN[t, r * w.B + a, h]))
    return ks, vs


def brute_attention(w, *, prefix=True, generated=True):
    G = w.Hq // w.Hkv
    scale = float(np.float32(w.scale))
    Q = to_f64(w.q)
    O = np.zeros((w.N_b, w.Hq, w.D))
    LSE = np.zeros((w.N_b, w.Hq))
    for r in range(w.R):
        for b in range(w.B):
            n = r * w.B + b
            for qh in range(w.Hq):
                h = qh // G
                ks, vs = beam_keys(w, r, b, h, prefix=prefix, generated=generated)
                q = list(Q[n, qh])
                if not ks:
                    O[n, qh] = 0.0
                    LSE[n, qh] = -math.inf
                    continue
                s = []
                for k in ks:
                    acc = 0.0
                    for d in range(w.D):
                        acc += q[d] * k[d]
                    s.append(scale * acc)
                m = max(s)
                e = [math.exp(x - m) for x in s]
                l = sum(e)
                for d in range(w.D):
                    O[n, qh, d] = sum(e[i] * vs[i][d] for i in range(len(ks))) / l
                LSE[n, qh] = m + math.log(l)
    return O, LSE
