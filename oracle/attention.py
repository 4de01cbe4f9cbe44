"""fp64 CPU oracle for staged beam-search decode attention.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no code
with the HIP library and imports nothing from it; it consumes the exact input
values (bf16 or fp32, upcast exactly to float64) the device is given.

What it computes (xGR page, "xGR: Atendimento de Recomendação Generativa
Eficiente em Escala", section 2.1 xAttention): every beam attends to the request's prompt
(the Shared cache, computed once at prefill) followed by the tokens generated
along that beam's own history (the Non-Shared cache, one token per decode
step). Splitting the computation into Shared / Non-Shared stages joined by an
online-softmax merge is exact in real arithmetic, so the oracle is the plain
definition: ONE softmax over each beam's full concatenated key sequence.

Readings of points the page leaves open:
  * the softmax scale is passed in (1/sqrt(D) by default);
  * a query head q uses kv head q // G, G = H_q / H_kv (grouped heads);
  * the unshared length L_r counts the current step's own token (append, then
    attend);
  * beam b's history is found by walking parent links backwards: the token of
    step L_r - 1 is beam b's own, the one of step t - 1 belongs to the parent
    (at step t) of the beam that owns step t; parents at step 0 are ignored;
  * an empty key sequence yields O = 0 and lse = -inf.

Outputs: O[n, q, :] (float64) and lse[n, q] = natural-log sum of exp(scores).
"""
from __future__ import annotations

import numpy as np


def _f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:  # bf16 bit pattern -> exact float64
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def lineage(parents: np.ndarray, r: int, B: int, L: int) -> np.ndarray:
    """anc[t, b] = the beam (request-local index) whose step-t token lies on
    beam b's history after L steps. Shape [L, B]."""
    anc = np.empty((L, B), dtype=np.int64)
    if L == 0:
        return anc
    anc[L - 1] = np.arange(B)
    for t in range(L - 1, 0, -1):
        anc[t - 1] = parents[t, r * B + anc[t]]
    return anc


def _attend_rows(qrows, kp, vp, kg, vg, scale):
    """One softmax over [prefix keys | generated keys] for a block of beams.

    qrows: [nb, G, D]; kp, vp: [P, D] shared by all rows; kg, vg: [nb, L, D]
    per beam. Returns O [nb, G, D], lse [nb, G].
    """
    nb, G, D = qrows.shape
    s_p = scale * np.matmul(qrows.reshape(nb * G, D), kp.T).reshape(nb, G, -1)
    s_g = scale * np.matmul(qrows, np.swapaxes(kg, 1, 2))          # [nb, G, L]
    s = np.concatenate([s_p, s_g], axis=-1)
    if s.shape[-1] == 0:
        return np.zeros((nb, G, D)), np.full((nb, G), -np.inf)
    m = s.max(axis=-1, keepdims=True)
    w = np.exp(s - m)
    l = w.sum(axis=-1)
    P = kp.shape[0]
    o = np.matmul(w[..., :P].reshape(nb * G, P), vp).reshape(nb, G, D)
    o += np.matmul(w[..., P:], vg)
    o /= l[..., None]
    return o, m[..., 0] + np.log(l)


def attention(w, *, include_prefix: bool = True, include_generated: bool = True,
              requests=None, heads=None, row_chunk: int = 64):
    """Decode attention for every beam and query head of workload ``w``.

    include_prefix=False gives the Non-Shared stage alone (attention over the
    generated tokens only); include_generated=False the Shared stage alone.
    requests / heads restrict the work (other outputs stay NaN).
    Returns (O [N_b, H_q, D] float64, lse [N_b, H_q] float64).
    """
    R, B, Hq, Hkv, D = w.R, w.B, w.Hq, w.Hkv, w.D
    G = Hq // Hkv
    scale = float(np.float32(w.scale))
    O = np.full((R * B, Hq, D), np.nan)
    LSE = np.full((R * B, Hq), np.nan)
    reqs = range(R) if requests is None else requests
    hs = range(Hkv) if heads is None else heads
    for r in reqs:
        P = int(w.prefix_len[r]) if include_prefix else 0
        L = int(w.unshared_len[r]) if include_generated else 0
        off = int(w.prefix_off[r])
        anc = lineage(w.parents, r, B, L)
        for h in hs:
            kp = _f64(w.k_shared[h, off:off + P])
            vp = _f64(w.v_shared[h, off:off + P])
            for b0 in range(0, B, row_chunk):
                b1 = min(B, b0 + row_chunk)
                beams = r * B + np.arange(b0, b1)
                qrows = _f64(w.q[beams, h * G:(h + 1) * G])
                # generated token t of beam b is the one step t wrote for beam anc[t, b]
                kg = np.empty((b1 - b0, L, D))
                vg = np.empty((b1 - b0, L, D))
                for t in range(L):
                    src = r * B + anc[t, b0:b1]
                    kg[:, t] = _f64(w.k_new[t, src, h])
                    vg[:, t] = _f64(w.v_new[t, src, h])
                o, lse = _attend_rows(qrows, kp, vp, kg, vg, scale)
                O[beams, h * G:(h + 1) * G] = o
                LSE[beams, h * G:(h + 1) * G] = lse
    return O, LSE


def attention_rows(w, rows, *, include_prefix=True, include_generated=True):
    """Decode attention for selected (beam n, query head q) pairs only.

    Every row gets the same single softmax over its own key sequence as in
    ``attention``; rows of one (request, kv head) share one upcast of that
    prompt's K/V and one call, so any rows of a full-size workload can be
    checked without computing the rest. Rows may repeat and come in any
    order. Returns O [len(rows), D], lse [len(rows)].
    """
    G = w.Hq // w.Hkv
    scale = float(np.float32(w.scale))
    O = np.empty((len(rows), w.D))
    LSE = np.empty(len(rows))
    groups = {}
    for i, (n, qh) in enumerate(rows):
        groups.setdefault((int(n) // w.B, int(qh) // G), []).append(i)
    for (r, h), idx in groups.items():
        P = int(w.prefix_len[r]) if include_prefix else 0
        L = int(w.unshared_len[r]) if include_generated else 0
        off = int(w.prefix_off[r])
        anc = lineage(w.parents, r, w.B, L)
        kp = _f64(w.k_shared[h, off:off + P])
        vp = _f64(w.v_shared[h, off:off + P])
        beams = [int(rows[i][0]) - r * w.B for i in idx]
        qrows = np.stack([_f64(w.q[int(rows[i][0]), int(rows[i][1])]) for i in idx])[:, None, :]
        kg = np.empty((len(idx), L, w.D))
        vg = np.empty((len(idx), L, w.D))
        for t in range(L):
            src = r * w.B + anc[t, beams]
            kg[:, t] = _f64(w.k_new[t, src, h])
            vg[:, t] = _f64(w.v_new[t, src, h])
        o, lse = _attend_rows(qrows, kp, vp, kg, vg, scale)
        O[idx] = o[:, 0]
        LSE[idx] = lse[:, 0]
    return O, LSE


def merge(o_a, lse_a, o_b, lse_b):
    """Log-sum-exp combine of two partial attentions over disjoint key sets
    (the page's Merge stage: online softmax over per-stage max/sum statistics).

    Each part is given as its normalized output and natural-log lse; a part
    over no keys has lse = -inf and contributes nothing. Both empty gives
    O = 0, lse = -inf.
    """
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    lse = np.logaddexp(lse_a, lse_b)
    with np.errstate(invalid="ignore"):
        wa = np.where(np.isneginf(lse_a), 0.0, np.exp(lse_a - lse))
        wb = np.where(np.isneginf(lse_b), 0.0, np.exp(lse_b - lse))
    o = wa[..., None] * o_a + wb[..., None] * o_b
    o = np.where(np.isneginf(lse)[..., None], 0.0, o)
    return o, lse


def merge_many(parts):
    """Combine any number of (O, lse) partials over disjoint key sets."""
    o, lse = parts[0]
    for o2, lse2 in parts[1:]:
        o, lse = merge(o, lse, o2, lse2)
    return o, lse
