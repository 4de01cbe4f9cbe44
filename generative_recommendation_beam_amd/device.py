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
                           key_groups=key_groups)
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

