"""Seeded synthetic inputs for staged beam-search decode attention.

This module draws random numbers, rounds them to the storage dtype and lays
them out in the device layouts the C-ABI documents. It holds none of the
attention arithmetic and imports neither the HIP binding nor the oracle; both
sides consume the arrays it returns.

Workload shapes follow the xGR page ("xGR: Atendimento de Recomendação Generativa
Eficiente em Escala"): long user-history prompts with short fixed-length outputs
(section 1, workload mismatch bullet), beam widths from 128 to 512 (section 1,
beam-search overhead bullet; section 4, scalability bullet), and prompts of a
few thousand tokens (section 4, memory bullet). The prefix-homogeneous batch
shape follows the Feather page ("Requests of a Feather Must Flock Together",
Results, prefix-sensitivity bullet), scaled down. The pages publish no tensor,
so every value here is synthetic.

Storage convention: bf16 tensors are held as ``np.uint16`` bit patterns
(round-to-nearest-even from float32 draws); fp32 tensors as ``np.float32``.
``to_f64`` upcasts either exactly.

Layouts (all row-major):
  q           [N_b][H_q][D]                 N_b = R * B, beam n = r * B + b
  k_shared    [H_kv][n_ptok][D]             request r owns tokens
  v_shared    [H_kv][n_ptok][D]               [prefix_off[r], prefix_off[r] + P_r)
  k_new       [T_steps][N_b][H_kv][D]       new token of beam n at step t
  v_new       [T_steps][N_b][H_kv][D]
  parents     [T_steps][N_b] int32          request-local parent beam, row 0 unused
  prefix_len  [R] int32, prefix_off [R] int64, unshared_len [R] int32 (final L_r)
  slot_base   [R] int64                     request r's slab in the unshared pool
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# Seed tags: one independent stream per kind of draw.
TAG_Q, TAG_KP, TAG_VP, TAG_KN, TAG_VN, TAG_PARENT, TAG_LEN, TAG_OUTLIER = range(8)


def _rng(seed_key, tag: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(list(seed_key) + [tag]))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    # 32-bit arithmetic suffices: for finite inputs the largest pattern,
    # 0xFF7FFFFF, plus the rounding bias stays below 2^32.
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    return ((bits + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(a: np.ndarray) -> np.ndarray:
    """Exact upcast of a storage array (bf16 bits or float32) to float64."""
    if a.dtype == np.uint16:
        return bf16_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits(x)
    return np.ascontiguousarray(x, dtype=np.float32)


@dataclass
class Workload:
    name: str
    dtype: str                      # "bf16" | "f32" (storage and input dtype)
    R: int
    B: int
    Hq: int
    Hkv: int
    D: int
    prefix_len: np.ndarray          # [R] int32
    prefix_off: np.ndarray          # [R] int64
    unshared_len: np.ndarray        # [R] int32, L_r after all steps
    T_max: int                      # slot-table row stride
    scale: np.float32
    q: np.ndarray
    k_shared: np.ndarray
    v_shared: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    parents: np.ndarray             # [T_steps][N_b] int32
    slot_base: np.ndarray           # [R] int64
    num_slots: int
    meta: dict = field(default_factory=dict)

    @property
    def N_b(self) -> int:
        return self.R * self.B

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def T_steps(self) -> int:
        return int(self.k_new.shape[0])

    @property
    def n_ptok(self) -> int:
        return int(self.k_shared.shape[1])

    def active(self, t: int) -> np.ndarray:
        """uint8 [R]: requests that take a generation step at step t."""
        return (self.unshared_len > t).astype(np.uint8)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4


def _normal(rng, shape, std, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _apply_outliers(x: np.ndarray, rng, frac: float, mult: float) -> np.ndarray:
    mask = rng.random(size=x.shape, dtype=np.float32) < np.float32(frac)
    x[mask] *= np.float32(mult)
    return x


def _zipf_parents(rng, shape, B, a):
    w = (np.arange(B, dtype=np.float64) + 1.0) ** (-a)
    w /= w.sum()
    return rng.choice(B, size=shape, p=w).astype(np.int32)


def make_workload(name: str, *, R: int, B: int, Hq: int, Hkv: int, D: int,
                  prefix_len, unshared_len, dtype: str = "bf16",
                  seed_key=(0, 0), qkv_std: float = 1.0, q_std: Optional[float] = None,
                  outlier_frac: float = 0.0, outlier_mult: float = 8.0,
                  parent_dist: str = "uniform", zipf_a: float = 1.1,
                  T_max: Optional[int] = None, scale: Optional[float] = None,
                  prefix_copies: Optional[np.ndarray] = None) -> Workload:
    """Build one seeded workload.

    prefix_len / unshared_len: int or per-request sequence.
    parent_dist: "uniform" | "zipf" | "identity".
    prefix_copies: optional [R] int array; request r then reads physical
      prefix ``prefix_copies[r]`` (several requests may alias one copy).
    """
    N_b = R * B
    P = np.broadcast_to(np.asarray(prefix_len, dtype=np.int32), (R,)).copy()
    L = np.broadcast_to(np.asarray(unshared_len, dtype=np.int32), (R,)).copy()
    T_steps = int(L.max()) if R else 0
    if T_max is None:
        T_max = max(T_steps, 1)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    scale = np.float32(scale)
    q_std = qkv_std if q_std is None else q_std

    if prefix_copies is None:
        prefix_off = np.zeros(R, dtype=np.int64)
        if R:
            prefix_off[1:] = np.cumsum(P.astype(np.int64))[:-1]
        n_ptok = int(P.sum())
    else:
        prefix_off = np.asarray(prefix_copies, dtype=np.int64) * int(P.max())
        n_ptok = int((np.max(prefix_copies) + 1) * int(P.max()))

    q = _normal(_rng(seed_key, TAG_Q), (N_b, Hq, D), q_std, dtype)
    kp = _normal(_rng(seed_key, TAG_KP), (Hkv, n_ptok, D), qkv_std, dtype)
    vp = _normal(_rng(seed_key, TAG_VP), (Hkv, n_ptok, D), qkv_std, dtype)
    kn = _normal(_rng(seed_key, TAG_KN), (T_steps, N_b, Hkv, D), qkv_std, dtype)
    vn = _normal(_rng(seed_key, TAG_VN), (T_steps, N_b, Hkv, D), qkv_std, dtype)
    if outlier_frac > 0:
        orng = _rng(seed_key, TAG_OUTLIER)
        for x in (kp, vp, kn, vn):
            _apply_outliers(x, orng, outlier_frac, outlier_mult)

    if parent_dist == "uniform":
        par = _rng(seed_key, TAG_PARENT).integers(0, B, size=(T_steps, N_b), dtype=np.int32)
    elif parent_dist == "zipf":
        par = _zipf_parents(_rng(seed_key, TAG_PARENT), (T_steps, N_b), B, zipf_a)
    elif parent_dist == "identity":
        par = np.tile(np.tile(np.arange(B, dtype=np.int32), R), (T_steps, 1))
    else:
        raise ValueError(parent_dist)
    if T_steps:
        par[0] = 0  # step 0 descends from the prompt; parents are ignored there

    slot_base = np.arange(R, dtype=np.int64) * (B * T_max)
    return Workload(name=name, dtype=dtype, R=R, B=B, Hq=Hq, Hkv=Hkv, D=D,
                    prefix_len=P, prefix_off=prefix_off, unshared_len=L, T_max=int(T_max),
                    scale=scale, q=_store(q, dtype), k_shared=_store(kp, dtype),
                    v_shared=_store(vp, dtype), k_new=_store(kn, dtype), v_new=_store(vn, dtype),
                    parents=par, slot_base=slot_base, num_slots=int(R * B * T_max),
                    meta=dict(seed_key=tuple(seed_key)))


# ----------------------------------------------------------------------------
# The five benchmark-shaped workloads. cfg ids: 1, 2, 3, "4A", "4B", 5.
# ----------------------------------------------------------------------------

CONFIG_IDS = (1, 2, 3, "4A", "4B", 5)
# Variants of config 4B (same values): the 64 single-sequence requests read
# the 4 physical prefixes of 4A through aliased offsets, in grouped or
# interleaved request order, or grouped with one request reading a private
# copy of its prefix (one divergent request).
CONFIG4_VARIANTS = ("4B2g", "4B2i", "4B2d")


def _cfg_seed_id(cfg) -> int:
    return {1: 1, 2: 2, 3: 3, "4A": 4, "4B": 4, "4B2g": 4, "4B2i": 4, "4B2d": 4, 5: 5}[cfg]


def config(cfg, layer: int = 0, *, unscaled: bool = False) -> Workload:
    """Synthetic stand-in for one benchmark configuration.

    unscaled=True redraws Q/K/V as plain N(0,1) at the same shape (used to make
    parity checks sensitive where the scaled draws give near-uniform softmax).
    """
    sk = (_cfg_seed_id(cfg), layer, 1 if unscaled else 0)
    if cfg == 1:
        return make_workload("cfg1_tiny_f32", R=1, B=4, Hq=4, Hkv=1, D=64,
                             prefix_len=256, unshared_len=2, dtype="f32", seed_key=sk)
    if cfg == 2:
        std = 1.0 if unscaled else 1.0 / np.sqrt(128.0)
        return make_workload("cfg2_gr_semantic_id", R=8, B=128, Hq=16, Hkv=4, D=128,
                             prefix_len=1024, unshared_len=3, seed_key=sk, qkv_std=std)
    if cfg == 3:
        L = _rng(sk, TAG_LEN).integers(1, 4, size=4).astype(np.int32)
        return make_workload("cfg3_wide_beam", R=4, B=512, Hq=32, Hkv=8, D=128,
                             prefix_len=2048, unshared_len=L, seed_key=sk, qkv_std=1.0,
                             outlier_frac=0.01, outlier_mult=8.0, parent_dist="zipf",
                             T_max=3)
    if cfg == "4A":
        return make_workload("cfg4A_prefix_homogeneous", R=4, B=16, Hq=32, Hkv=8, D=128,
                             prefix_len=4096, unshared_len=512, seed_key=sk,
                             parent_dist="identity")
    if cfg == "4B":
        a = config("4A", layer, unscaled=unscaled)
        return as_distinct_prefixes(a, "cfg4B_prefix_heterogeneous")
    if cfg in CONFIG4_VARIANTS:
        a = config("4A", layer, unscaled=unscaled)
        order = "interleaved" if cfg == "4B2i" else "grouped"
        return as_aliased_prefixes(a, f"cfg{cfg}_prefix_aliased_{order}", order=order,
                                   divergent=(cfg == "4B2d"))
    if cfg == 5:
        std = 1.0 if unscaled else 1.0 / np.sqrt(128.0)
        return make_workload("cfg5_long_history", R=16, B=256, Hq=64, Hkv=8, D=128,
                             prefix_len=16384, unshared_len=8, seed_key=sk, qkv_std=std)
    raise ValueError(f"unknown config {cfg!r}")


def as_distinct_prefixes(w: Workload, name: str) -> Workload:
    """Re-express each beam of ``w`` as its own request with beam width 1.

    Beam n = r * B + b of ``w`` becomes request n, reading a private physical
    copy of its group's prefix. Values are identical, so outputs must match.
    Requires identity parents (every sequence keeps its own history).
    """
    B, R = w.B, w.R
    N_b = w.N_b
    Pmax = int(w.prefix_len.max())
    ks = np.empty((w.Hkv, N_b * Pmax, w.D), dtype=w.k_shared.dtype)
    vs = np.empty_like(ks)
    for n in range(N_b):
        r = n // B
        o = int(w.prefix_off[r])
        ks[:, n * Pmax:n * Pmax + int(w.prefix_len[r])] = w.k_shared[:, o:o + int(w.prefix_len[r])]
        vs[:, n * Pmax:n * Pmax + int(w.prefix_len[r])] = w.v_shared[:, o:o + int(w.prefix_len[r])]
    P = np.repeat(w.prefix_len, B)
    L = np.repeat(w.unshared_len, B)
    T_max = w.T_max
    return Workload(name=name, dtype=w.dtype, R=N_b, B=1, Hq=w.Hq, Hkv=w.Hkv, D=w.D,
                    prefix_len=P.astype(np.int32),
                    prefix_off=np.arange(N_b, dtype=np.int64) * Pmax,
                    unshared_len=L.astype(np.int32), T_max=T_max, scale=w.scale,
                    q=w.q, k_shared=ks, v_shared=vs, k_new=w.k_new, v_new=w.v_new,
                    parents=np.zeros_like(w.parents),
                    slot_base=np.arange(N_b, dtype=np.int64) * T_max,
                    num_slots=N_b * T_max, meta=dict(w.meta, derived_from=w.name))


def as_aliased_prefixes(w: Workload, name: str, order: str = "grouped",
                        divergent: bool = False) -> Workload:
    """Re-express each beam of ``w`` as its own request with beam width 1,
    every request of a group reading the group's one physical prefix (the
    prompt offsets alias).

    order "grouped": request n is sequence n (a group's requests are
    consecutive); "interleaved": request n belongs to group n % R, so
    consecutive requests read different prefixes. divergent: request 0 reads
    a private physical copy of its prefix instead. Values are unchanged, so
    request n's output equals that of sequence meta["seq_of_request"][n] of
    ``w``. Requires identity parents.
    """
    B, R = w.B, w.R
    N_b = w.N_b
    n = np.arange(N_b)
    if order == "grouped":
        seq = n
    elif order == "interleaved":
        seq = (n % R) * B + n // R
    else:
        raise ValueError(f"unknown order {order!r}")
    grp = seq // B
    P = w.prefix_len[grp].astype(np.int32)
    off = w.prefix_off[grp].astype(np.int64)
    ks, vs = w.k_shared, w.v_shared
    if divergent:
        o0, p0 = int(off[0]), int(P[0])
        off = off.copy()
        off[0] = ks.shape[1]
        ks = np.concatenate([ks, ks[:, o0:o0 + p0]], axis=1)
        vs = np.concatenate([vs, vs[:, o0:o0 + p0]], axis=1)
    T_max = w.T_max
    return Workload(name=name, dtype=w.dtype, R=N_b, B=1, Hq=w.Hq, Hkv=w.Hkv, D=w.D,
                    prefix_len=P, prefix_off=off,
                    unshared_len=w.unshared_len[grp].astype(np.int32), T_max=T_max, scale=w.scale,
                    q=w.q[seq], k_shared=ks, v_shared=vs, k_new=w.k_new[:, seq], v_new=w.v_new[:, seq],
                    parents=np.zeros_like(w.parents),
                    slot_base=np.arange(N_b, dtype=np.int64) * T_max,
                    num_slots=N_b * T_max,
                    meta=dict(w.meta, derived_from=w.name, seq_of_request=seq.tolist()))


@dataclass
class TopKInput:
    """One decode step's beam-search candidate pools, per request.

    beam_score [R][BW] f32: cumulative log-probability of each live beam
    (descending in b, as the previous selection leaves them); logprob
    [R][BW][K] f32: each beam's K best next-token log-probabilities, sorted
    descending along K (equal values keep their vocabulary order); token
    [R][BW][K] int32: the matching token ids; n_out: beams to keep.
    """
    name: str
    beam_score: np.ndarray
    logprob: np.ndarray
    token: np.ndarray
    n_out: int
    meta: dict = field(default_factory=dict)

    @property
    def R(self) -> int:
        return int(self.logprob.shape[0])

    @property
    def BW(self) -> int:
        return int(self.logprob.shape[1])

    @property
    def K(self) -> int:
        return int(self.logprob.shape[2])


def make_topk(name: str, *, R: int, BW: int, K: int, n_out: Optional[int] = None,
              seed_key=(0, 0), dist: str = "softmax", vocab: int = 8192, step: int = 3,
              logit_std: float = 2.0) -> TopKInput:
    """Seeded candidate pools.

    dist:
      "softmax": per beam, logits ~ N(0, logit_std^2) over `vocab` tokens,
                 log-softmax (float64, then float32), the K largest kept in
                 descending order; beam scores are the sum of `step` earlier
                 such picks plus noise, sorted descending;
      "ties":    like softmax, but log-probs and beam scores are rounded to
                 multiples of 1/4 so that many candidate scores tie exactly;
      "masked":  like softmax, with a random tail of each beam set to -inf
                 (tokens a validity mask removed);
      "equal":   every log-prob and beam score is the same value.
    """
    n_out = BW if n_out is None else n_out
    rng = np.random.default_rng(np.random.SeedSequence([0x70B, *[int(x) for x in seed_key]]))
    if dist == "equal":
        lp = np.full((R, BW, K), -1.5, dtype=np.float32)
        bs = np.full((R, BW), -4.0, dtype=np.float32)
        tok = np.broadcast_to(np.arange(K, dtype=np.int32), (R, BW, K)).copy()
        return TopKInput(name, bs, lp, tok, n_out, dict(dist=dist))
    lp = np.empty((R, BW, K), dtype=np.float32)
    tok = np.empty((R, BW, K), dtype=np.int32)
    for r in range(R):
        logits = rng.standard_normal(size=(BW, vocab)) * logit_std
        logits -= logits.max(axis=1, keepdims=True)
        lsm = logits - np.log(np.exp(logits).sum(axis=1, keepdims=True))
        order = np.argsort(-lsm, axis=1, kind="stable")[:, :K]
        lp[r] = np.take_along_axis(lsm, order, axis=1).astype(np.float32)
        tok[r] = order.astype(np.int32)
    base = np.float32(step) * lp[:, :, 0].mean(axis=1, keepdims=True)
    bs = (base + rng.standard_normal(size=(R, BW)).astype(np.float32)).astype(np.float32)
    bs = -np.sort(-bs, axis=1)
    if dist == "ties":
        # rounding is monotone, so each beam's row stays sorted (with ties)
        lp = (np.round(lp * 4.0) / 4.0).astype(np.float32)
        bs = (np.round(bs * 4.0) / 4.0).astype(np.float32)
    elif dist == "masked":
        cut = rng.integers(1, K + 1, size=(R, BW))
        for r in range(R):
            for b in range(BW):
                lp[r, b, cut[r, b]:] = -np.inf
    elif dist != "softmax":
        raise ValueError(dist)
    return TopKInput(name, bs.astype(np.float32), lp, tok, n_out, dict(dist=dist))
