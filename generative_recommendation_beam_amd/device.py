"""Put a synthetic workload into device memory and drive the C-ABI on it.

PyTorch provides device memory and the stream; every computation is a call
into libxattn.so. The Non-Shared pool and slot tables are built on the
device by ``xattn_cache_append``, one call per decode step, exactly as a
serving loop would.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import xattn
from .inputs import Workload


def _to_dev(a: np.ndarray, device, dtype: Optional[str] = None) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


@dataclass
class DeviceWorkload:
    w: Workload
    dims: xattn.Dims
    q: torch.Tensor
    k_shared: torch.Tensor
    v_shared: torch.Tensor
    prefix_off: torch.Tensor
    prefix_len: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    parents: torch.Tensor
    active: torch.Tensor
    slot_base: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    table: torch.Tensor
    unshared_len: torch.Tensor

    @property
    def rows(self) -> int:
        return self.w.N_b * self.w.Hq


def upload(w: Workload, device="cuda", *, prefix_splits=0, unshared_splits=0,
           rows_per_block=0, pipeline_stages=0, key_groups=0, table_fill: int = -1) -> DeviceWorkload:
    dims = xattn.make_dims(R=w.R, B=w.B, Hq=w.Hq, Hkv=w.Hkv, D=w.D,
                           max_prefix_len=int(w.prefix_len.max()) if w.R else 0,
                           max_unshared_len=w.T_max,
                           dtype=xattn.XATTN_BF16 if w.dtype == "bf16" else xattn.XATTN_F32,
                           num_slots=w.num_slots, num_prefix_tokens=w.n_ptok, scale=w.scale,
                           prefix_splits=prefix_splits, unshared_splits=unshared_splits,
                           rows_per_block=rows_per_block, pipeline_stages=pipeline_stages,
                           key_groups=key_groups,
                           prompts_disjoint=xattn.prompts_disjoint(w.prefix_off, w.prefix_len))
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    T = w.T_steps
    act = np.stack([w.active(t) for t in range(T)]) if T else np.zeros((0, w.R), np.uint8)
    return DeviceWorkload(
        w=w, dims=dims, q=_to_dev(w.q, device), k_shared=_to_dev(w.k_shared, device),
        v_shared=_to_dev(w.v_shared, device),
        prefix_off=torch.from_numpy(w.prefix_off.astype(np.int64)).to(device),
        prefix_len=torch.from_numpy(w.prefix_len.astype(np.int32)).to(device),
        k_new=_to_dev(w.k_new, device), v_new=_to_dev(w.v_new, device),
        parents=torch.from_numpy(w.parents.astype(np.int32)).to(device),
        active=torch.from_numpy(act.astype(np.uint8)).to(device),
        slot_base=torch.from_numpy(w.slot_base.astype(np.int64)).to(device),
        k_pool=torch.zeros((max(w.num_slots, 1), w.Hkv, w.D), dtype=tdt, device=device),
        v_pool=torch.zeros((max(w.num_slots, 1), w.Hkv, w.D), dtype=tdt, device=device),
        table=torch.full((max(w.N_b, 1), w.T_max), table_fill, dtype=torch.int32, device=device),
        unshared_len=torch.zeros(max(w.R, 1), dtype=torch.int32, device=device),
    )


def append_step(d: DeviceWorkload, t: int, *, table_in=None, table_out=None, stream=None):
    table_in = d.table if table_in is None else table_in
    table_out = d.table if table_out is None else table_out
    xattn.cache_append(d.dims, d.k_new[t], d.v_new[t], d.parents[t], d.slot_base, d.active[t],
                       d.k_pool, d.v_pool, table_in, table_out, d.unshared_len, stream=stream)


def build_cache(d: DeviceWorkload, stream=None):
    """Run every decode step's append on the device (in place)."""
    for t in range(d.w.T_steps):
        append_step(d, t, stream=stream)


def alloc_outputs(d: DeviceWorkload, which: int = 2):
    dev = d.q.device
    o = torch.empty((max(d.rows, 1), d.w.D), dtype=torch.float32, device=dev)
    lse = torch.empty(max(d.rows, 1), dtype=torch.float32, device=dev)
    nbytes = xattn.workspace_size(d.dims, which)
    ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=dev)  # counters start at zero
    return o, lse, ws, nbytes


def decode(d: DeviceWorkload, o, lse, ws, nbytes, stream=None):
    xattn.decode(d.dims, d.q, d.k_shared, d.v_shared, d.prefix_off, d.prefix_len, d.k_pool,
                 d.v_pool, d.table, d.unshared_len, o, lse, ws if nbytes else None, nbytes,
                 stream=stream)


def shared_stage(d: DeviceWorkload, o, lse, ws, nbytes, stream=None):
    xattn.shared_stage(d.dims, d.q, d.k_shared, d.v_shared, d.prefix_off, d.prefix_len, o, lse,
                       ws if nbytes else None, nbytes, stream=stream)


def unshared_stage(d: DeviceWorkload, o, lse, ws, nbytes, stream=None):
    xattn.unshared_stage(d.dims, d.q, d.k_pool, d.v_pool, d.table, d.unshared_len, o, lse,
                         ws if nbytes else None, nbytes, stream=stream)


def prepare_step(d: DeviceWorkload):
    """Cache state one step before the end: every decode step but the last is
    appended (in place into d.table). Returns (table_in, table_out, t_last):
    the step appends step t_last's tokens from table_in into table_out and
    decodes on table_out; t_last is None when there are no generated tokens.
    Restoring d.unshared_len to its value here makes the step repeatable."""
    T = d.w.T_steps
    for t in range(max(T - 1, 0)):
        append_step(d, t)
    table_out = d.table.clone()
    return d.table, table_out, (T - 1 if T > 0 else None)


def layer_step(d: DeviceWorkload, o, lse, ws, nbytes, table_in, table_out, t_last,
               decode_begin=None, decode_end=None):
    """xattn_layer_step of one layer: append step t_last (if any), then decode."""
    app = {}
    if t_last is not None:
        app = dict(k_new=d.k_new[t_last], v_new=d.v_new[t_last], parent=d.parents[t_last],
                   slot_base=d.slot_base, active=d.active[t_last], table_in=table_in)
    return xattn.layer_step(d.dims, q=d.q, k_shared=d.k_shared, v_shared=d.v_shared,
                            prefix_off=d.prefix_off, prefix_len=d.prefix_len, k_pool=d.k_pool,
                            v_pool=d.v_pool, table_out=table_out, unshared_len=d.unshared_len,
                            o=o, lse=lse, workspace=ws if nbytes else None,
                            workspace_bytes=nbytes, decode_begin=decode_begin,
                            decode_end=decode_end, **app)



# ---- PagedAttention-style comparison layout ----
PAGED_BLOCK = 16


@dataclass
class PagedCache:
    """The same caches as a DeviceWorkload, laid out the PagedAttention way:
    16-token blocks [num_blocks][H_kv][16][D]; a request's full prompt blocks
    are shared by its beams, and each beam owns blocks holding the prompt's
    last partial block followed by its own generated tokens. `tail_block[n]`
    is beam n's last block, `spare` one spare block per beam (the copy a
    branching beam makes lands there)."""
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor
    seq_len: torch.Tensor
    max_seq_len: int
    tail_block: torch.Tensor
    parent_tail: torch.Tensor
    spare: torch.Tensor


def build_paged(d: DeviceWorkload, table=None) -> PagedCache:
    """Build the paged layout from d's prompt KV and (already built) Non-Shared
    cache, reading generated tokens through `table` (default d.table). Data
    preparation for the baseline: index arithmetic on the host, gathers on
    the device."""
    w = d.w
    BS = PAGED_BLOCK
    P = w.prefix_len.astype(np.int64)
    L = w.unshared_len.astype(np.int64)
    table = (d.table if table is None else table).cpu().numpy()
    n_blocks = 0
    shared = []
    for r in range(w.R):
        shared.append(list(range(n_blocks, n_blocks + int(P[r] // BS))))
        n_blocks += int(P[r] // BS)
    rows, seq = [], []
    src_prompt, src_slot = [], []   # per cache token: prompt token index (h-free) or pool slot
    priv_first = []
    for r in range(w.R):
        tail = int(P[r] % BS)
        for b in range(w.B):
            n = r * w.B + b
            ntok = tail + int(L[r])
            nb = (ntok + BS - 1) // BS
            priv = list(range(n_blocks, n_blocks + nb))
            n_blocks += nb
            priv_first.append(priv)
            rows.append(shared[r] + priv)
            seq.append(int(P[r] + L[r]))
    max_blocks = max([len(x) for x in rows] + [1])
    bt = np.zeros((w.N_b, max_blocks), np.int32)
    for n, row in enumerate(rows):
        bt[n, :len(row)] = row
    spare0 = n_blocks
    total_blocks = n_blocks + w.N_b
    # token map: for every (block, i) which source fills it
    kind = np.zeros((total_blocks, BS), np.int8)       # 0 none, 1 prompt, 2 pool
    idx = np.zeros((total_blocks, BS), np.int64)
    for r in range(w.R):
        off = int(w.prefix_off[r])
        for j, blk in enumerate(shared[r]):
            kind[blk] = 1
            idx[blk] = off + j * BS + np.arange(BS)
        tail = int(P[r] % BS)
        for b in range(w.B):
            n = r * w.B + b
            toks = [(1, off + int(P[r]) - tail + i) for i in range(tail)]
            toks += [(2, int(table[n, t])) for t in range(int(L[r]))]
            for k, (kd, ix) in enumerate(toks):
                blk = priv_first[n][k // BS]
                kind[blk, k % BS] = kd
                idx[blk, k % BS] = ix
    dev = d.q.device
    tdt = d.k_shared.dtype
    kc = torch.zeros((total_blocks, w.Hkv, BS, w.D), dtype=tdt, device=dev)
    vc = torch.zeros_like(kc)
    kind_t = torch.from_numpy(kind).to(dev)
    idx_t = torch.from_numpy(idx).to(dev)
    for h in range(w.Hkv):
        m1 = kind_t == 1
        if bool(m1.any()):
            kc[:, h][m1] = d.k_shared[h][idx_t[m1]]
            vc[:, h][m1] = d.v_shared[h][idx_t[m1]]
        m2 = kind_t == 2
        if bool(m2.any()):
            kc[:, h][m2] = d.k_pool[idx_t[m2], h]
            vc[:, h][m2] = d.v_pool[idx_t[m2], h]
    tail_block = np.array([row[-1] if row else 0 for row in rows], np.int32)
    # the block a beam's tail was copied from at the last step: its parent's
    t_last = w.T_steps - 1
    parent = np.arange(w.N_b) if t_last < 1 else \
        (np.arange(w.N_b) // w.B) * w.B + w.parents[t_last]
    return PagedCache(k_cache=kc, v_cache=vc, block_table=torch.from_numpy(bt).to(dev),
                      seq_len=torch.tensor(seq, dtype=torch.int32, device=dev), max_seq_len=max(seq + [0]),
                      tail_block=torch.from_numpy(tail_block).to(dev),
                      parent_tail=torch.from_numpy(tail_block[parent].astype(np.int32)).to(dev),
                      spare=torch.arange(spare0, spare0 + w.N_b, dtype=torch.int32, device=dev))


def paged_decode(d: DeviceWorkload, pc: PagedCache, o, lse, ws=None, nbytes=0, stream=None):
    xattn.paged_decode(d.dims, pc.max_seq_len, d.q, pc.k_cache, pc.v_cache, pc.block_table, pc.seq_len, o,
                       lse, ws if nbytes else None, nbytes, stream=stream)
