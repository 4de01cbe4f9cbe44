"""ctypes binding of the xattn C-ABI (argument marshalling only).

Every step of the path runs in the HIP library ``libxattn.so``; this module
only turns torch tensors into device pointers, passes the current HIP stream
and raises on a non-OK status. If the library is missing, importing the
binding's functions raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libxattn.so")

XATTN_OK, XATTN_ERR_INVALID_ARG, XATTN_ERR_UNSUPPORTED, XATTN_ERR_WORKSPACE, XATTN_ERR_HIP = range(5)
XATTN_F32, XATTN_BF16 = 0, 1

EXPORTED = ("xattn_workspace_size", "xattn_get_plan", "xattn_shared_stage", "xattn_unshared_stage",
            "xattn_merge", "xattn_decode", "xattn_cache_append", "xattn_append_decode", "xattn_beam_topk",
            "xattn_paged_workspace_size", "xattn_paged_decode", "xattn_paged_copy_blocks",
            "xattn_cht_create", "xattn_cht_destroy", "xattn_cht_insert", "xattn_cht_best",
            "xattn_cht_admit", "xattn_cht_complete", "xattn_cht_form_batch", "xattn_step_graph_create",
            "xattn_step_graph_launch", "xattn_step_graph_destroy", "xattn_stream_read", "xattn_append_decode_static",
            "xattn_status_string")


class Dims(ctypes.Structure):
    _fields_ = [("num_requests", ctypes.c_int32), ("beam_width", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("max_prefix_len", ctypes.c_int32),
                ("max_unshared_len", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("num_slots", ctypes.c_int64), ("num_prefix_tokens", ctypes.c_int64),
                ("scale", ctypes.c_float), ("prefix_splits", ctypes.c_int32),
                ("unshared_splits", ctypes.c_int32), ("rows_per_block", ctypes.c_int32),
                ("pipeline_stages", ctypes.c_int32), ("key_groups", ctypes.c_int32),
                ("prompts_disjoint", ctypes.c_int32)]


class Plan(ctypes.Structure):
    _fields_ = [("rows_per_block", ctypes.c_int32), ("row_tiles", ctypes.c_int32),
                ("prefix_splits", ctypes.c_int32), ("prefix_chunk", ctypes.c_int32),
                ("unshared_splits", ctypes.c_int32), ("unshared_chunk", ctypes.c_int32),
                ("partials", ctypes.c_int32), ("mfma", ctypes.c_int32),
                ("launches", ctypes.c_int32), ("pipeline_stages", ctypes.c_int32),
                ("key_groups", ctypes.c_int32)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


P_ = ctypes.c_void_p


class LayerStep(ctypes.Structure):
    """One layer of a captured decode step (xattn_layer_step)."""
    _fields_ = [("dims", Dims), ("k_new", P_), ("v_new", P_), ("parent", P_), ("slot_base", P_),
                ("active", P_), ("table_in", P_), ("table_out", P_), ("unshared_len", P_),
                ("q", P_), ("k_shared", P_), ("v_shared", P_), ("prefix_off", P_),
                ("prefix_len", P_), ("k_pool", P_), ("v_pool", P_), ("o", P_), ("lse", P_),
                ("workspace", P_), ("workspace_bytes", ctypes.c_size_t), ("decode_begin", P_),
                ("decode_end", P_)]


class BeamSelect(ctypes.Structure):
    """The survivor selection that opens a captured step (xattn_beam_select)."""
    _fields_ = [("num_requests", ctypes.c_int32), ("beam_width", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("n_out", ctypes.c_int32), ("beam_score", P_),
                ("logprob", P_), ("token", P_), ("parent", P_), ("token_out", P_),
                ("score_out", P_)]


class XattnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


_lib = None


def lib():
    """Load libxattn.so (built in-tree); raise loudly if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"xattn HIP library not built: {LIB_PATH} is missing "
                           "(run __graft_entry__.build() or python -m "
                           "generative_recommendation_beam_amd.build)")
    L = ctypes.CDLL(LIB_PATH, mode=os.RTLD_NOW | os.RTLD_LOCAL)
    P = ctypes.c_void_p
    pd = ctypes.POINTER(Dims)
    L.xattn_status_string.restype = ctypes.c_char_p
    L.xattn_status_string.argtypes = [ctypes.c_int]
    L.xattn_workspace_size.restype = ctypes.c_int
    L.xattn_workspace_size.argtypes = [pd, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
    L.xattn_get_plan.restype = ctypes.c_int
    L.xattn_get_plan.argtypes = [pd, ctypes.c_int, ctypes.POINTER(Plan)]
    L.xattn_shared_stage.restype = ctypes.c_int
    L.xattn_shared_stage.argtypes = [pd, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.xattn_unshared_stage.restype = ctypes.c_int
    L.xattn_unshared_stage.argtypes = [pd, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.xattn_merge.restype = ctypes.c_int
    L.xattn_merge.argtypes = [ctypes.c_int64, ctypes.c_int32, P, P, P, P, P, P, P]
    L.xattn_decode.restype = ctypes.c_int
    L.xattn_decode.argtypes = [pd, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.xattn_cache_append.restype = ctypes.c_int
    L.xattn_cache_append.argtypes = [pd, P, P, P, P, P, P, P, P, P, P, P]
    L.xattn_append_decode.restype = ctypes.c_int
    L.xattn_append_decode.argtypes = [pd] + [P] * 18 + [ctypes.c_size_t, P]
    L.xattn_paged_workspace_size.restype = ctypes.c_int
    L.xattn_paged_workspace_size.argtypes = [pd, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
    L.xattn_paged_decode.restype = ctypes.c_int
    L.xattn_paged_decode.argtypes = [pd, ctypes.c_int32, P, P, P, P, ctypes.c_int32, P, P, P, P,
                                     ctypes.c_size_t, P]
    L.xattn_paged_copy_blocks.restype = ctypes.c_int
    L.xattn_paged_copy_blocks.argtypes = [pd, P, P, P, P, ctypes.c_int32, P]
    i64 = ctypes.c_int64
    L.xattn_cht_create.restype = ctypes.c_int
    L.xattn_cht_create.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p)]
    L.xattn_cht_destroy.restype = ctypes.c_int
    L.xattn_cht_destroy.argtypes = [P]
    L.xattn_cht_insert.restype = ctypes.c_int
    L.xattn_cht_insert.argtypes = [P, i64, P, i64]
    L.xattn_cht_best.restype = ctypes.c_int
    L.xattn_cht_best.argtypes = [P, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.xattn_cht_admit.restype = ctypes.c_int
    L.xattn_cht_admit.argtypes = [P, i64]
    L.xattn_cht_complete.restype = ctypes.c_int
    L.xattn_cht_complete.argtypes = [P, i64]
    L.xattn_cht_form_batch.restype = ctypes.c_int
    L.xattn_cht_form_batch.argtypes = [P, ctypes.c_int32, i64, P, ctypes.POINTER(ctypes.c_int32)]
    L.xattn_beam_topk.restype = ctypes.c_int
    L.xattn_beam_topk.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                  P, P, P, P, P, P, P]
    L.xattn_step_graph_create.restype = ctypes.c_int
    L.xattn_step_graph_create.argtypes = [ctypes.POINTER(BeamSelect), ctypes.POINTER(LayerStep),
                                          ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p)]
    L.xattn_step_graph_launch.restype = ctypes.c_int
    L.xattn_step_graph_launch.argtypes = [P, P]
    L.xattn_step_graph_destroy.restype = ctypes.c_int
    L.xattn_step_graph_destroy.argtypes = [P]
    L.xattn_append_decode_static.restype = ctypes.c_int
    L.xattn_append_decode_static.argtypes = [pd] + [P] * 17 + [P]
    L.xattn_stream_read.restype = ctypes.c_int
    L.xattn_stream_read.argtypes = [P, ctypes.c_size_t, P, P]
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().xattn_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != XATTN_OK:
        raise XattnError(status, where)


def _ptr(t):
    """Device (or host) address of a tensor / None -> NULL."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def make_dims(*, R, B, Hq, Hkv, D, max_prefix_len, max_unshared_len, dtype, num_slots,
              num_prefix_tokens, scale, prefix_splits=0, unshared_splits=0, rows_per_block=0,
              pipeline_stages=0, key_groups=0, prompts_disjoint=0) -> Dims:
    return Dims(int(R), int(B), int(Hq), int(Hkv), int(D), int(max_prefix_len),
                int(max_unshared_len), int(dtype), int(num_slots), int(num_prefix_tokens),
                float(scale), int(prefix_splits), int(unshared_splits), int(rows_per_block),
                int(pipeline_stages), int(key_groups), int(prompts_disjoint))


def prompts_disjoint(prefix_off, prefix_len) -> bool:
    """True when no two requests' prompt ranges [off, off + len) overlap
    (empty ranges overlap nothing): the guarantee behind the dims hint."""
    rs = sorted((int(o), int(o) + int(n)) for o, n in zip(prefix_off, prefix_len) if int(n) > 0)
    return all(a[1] <= b[0] for a, b in zip(rs, rs[1:]))


def workspace_size(dims: Dims, which: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().xattn_workspace_size(ctypes.byref(dims), int(which), ctypes.byref(n)),
           "xattn_workspace_size")
    return int(n.value)


def get_plan(dims: Dims, which: int) -> dict:
    p = Plan()
    _check(lib().xattn_get_plan(ctypes.byref(dims), int(which), ctypes.byref(p)), "xattn_get_plan")
    return p.as_dict()


def shared_stage(dims, q, k_shared, v_shared, prefix_off, prefix_len, o, lse, workspace=None,
                 workspace_bytes=0, stream=None):
    _check(lib().xattn_shared_stage(ctypes.byref(dims), _ptr(q), _ptr(k_shared), _ptr(v_shared),
                                    _ptr(prefix_off), _ptr(prefix_len), _ptr(o), _ptr(lse),
                                    _ptr(workspace), int(workspace_bytes), _stream(stream)),
           "xattn_shared_stage")


def unshared_stage(dims, q, k_pool, v_pool, slot_table, unshared_len, o, lse, workspace=None,
                   workspace_bytes=0, stream=None):
    _check(lib().xattn_unshared_stage(ctypes.byref(dims), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                      _ptr(slot_table), _ptr(unshared_len), _ptr(o), _ptr(lse),
                                      _ptr(workspace), int(workspace_bytes), _stream(stream)),
           "xattn_unshared_stage")


def merge(rows, head_dim, o_a, lse_a, o_b, lse_b, o_out, lse_out=None, stream=None):
    _check(lib().xattn_merge(int(rows), int(head_dim), _ptr(o_a), _ptr(lse_a), _ptr(o_b),
                             _ptr(lse_b), _ptr(o_out), _ptr(lse_out), _stream(stream)),
           "xattn_merge")


def decode(dims, q, k_shared, v_shared, prefix_off, prefix_len, k_pool, v_pool, slot_table,
           unshared_len, o, lse=None, workspace=None, workspace_bytes=0, stream=None):
    _check(lib().xattn_decode(ctypes.byref(dims), _ptr(q), _ptr(k_shared), _ptr(v_shared),
                              _ptr(prefix_off), _ptr(prefix_len), _ptr(k_pool), _ptr(v_pool),
                              _ptr(slot_table), _ptr(unshared_len), _ptr(o), _ptr(lse),
                              _ptr(workspace), int(workspace_bytes), _stream(stream)),
           "xattn_decode")


def cache_append(dims, k_new, v_new, parent, slot_base, active, k_pool, v_pool, table_in,
                 table_out, unshared_len, stream=None):
    _check(lib().xattn_cache_append(ctypes.byref(dims), _ptr(k_new), _ptr(v_new), _ptr(parent),
                                    _ptr(slot_base), _ptr(active), _ptr(k_pool), _ptr(v_pool),
                                    _ptr(table_in), _ptr(table_out), _ptr(unshared_len),
                                    _stream(stream)),
           "xattn_cache_append")


def append_decode(dims, q, k_shared, v_shared, prefix_off, prefix_len, k_new, v_new, parent, slot_base,
                  active, k_pool, v_pool, table_in, table_out, unshared_len, o, lse=None, workspace=None,
                  workspace_bytes=0, stream=None):
    _check(lib().xattn_append_decode(ctypes.byref(dims), _ptr(q), _ptr(k_shared), _ptr(v_shared),
                                     _ptr(prefix_off), _ptr(prefix_len), _ptr(k_new), _ptr(v_new),
                                     _ptr(parent), _ptr(slot_base), _ptr(active), _ptr(k_pool),
                                     _ptr(v_pool), _ptr(table_in), _ptr(table_out), _ptr(unshared_len),
                                     _ptr(o), _ptr(lse), _ptr(workspace), int(workspace_bytes),
                                     _stream(stream)),
           "xattn_append_decode")


def stream_read(src, sink, nbytes=None, stream=None):
    """Measurement utility: read `nbytes` (default: all) of tensor src once."""
    nbytes = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    _check(lib().xattn_stream_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)), "xattn_stream_read")


def append_decode_static(dims, q, k_shared, v_shared, prefix_off, prefix_len, k_new, v_new, parent, slot_base,
                         active, k_pool, v_pool, table_in, table_out, unshared_len, o, lse=None, stream=None):
    """xattn_append_decode with the library's fixed device workspace (no
    workspace argument; calls on one GPU must not overlap)."""
    _check(lib().xattn_append_decode_static(ctypes.byref(dims), _ptr(q), _ptr(k_shared), _ptr(v_shared),
                                            _ptr(prefix_off), _ptr(prefix_len), _ptr(k_new), _ptr(v_new),
                                            _ptr(parent), _ptr(slot_base), _ptr(active), _ptr(k_pool),
                                            _ptr(v_pool), _ptr(table_in), _ptr(table_out), _ptr(unshared_len),
                                            _ptr(o), _ptr(lse), _stream(stream)),
           "xattn_append_decode_static")


def paged_workspace_size(dims, max_seq_len) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().xattn_paged_workspace_size(ctypes.byref(dims), int(max_seq_len), ctypes.byref(n)),
           "xattn_paged_workspace_size")
    return int(n.value)


def paged_decode(dims, max_seq_len, q, k_cache, v_cache, block_table, seq_len, o, lse=None,
                 workspace=None, workspace_bytes=0, stream=None):
    _check(lib().xattn_paged_decode(ctypes.byref(dims), int(max_seq_len), _ptr(q), _ptr(k_cache),
                                    _ptr(v_cache), _ptr(block_table), int(block_table.shape[1]),
                                    _ptr(seq_len), _ptr(o), _ptr(lse), _ptr(workspace),
                                    int(workspace_bytes), _stream(stream)),
           "xattn_paged_decode")


def paged_copy_blocks(dims, k_cache, v_cache, src, dst, stream=None):
    _check(lib().xattn_paged_copy_blocks(ctypes.byref(dims), _ptr(k_cache), _ptr(v_cache), _ptr(src),
                                         _ptr(dst), int(src.shape[0]), _stream(stream)),
           "xattn_paged_copy_blocks")


class Cht:
    """Host-side batch former (xattn_cht_*): cumulative block hashes, a
    working set of the active batch and a min-heap by missing blocks."""

    def __init__(self, block_size: int):
        h = ctypes.c_void_p(None)
        _check(lib().xattn_cht_create(int(block_size), ctypes.byref(h)), "xattn_cht_create")
        self._h = h

    def insert(self, rid: int, tokens) -> None:
        arr = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        _check(lib().xattn_cht_insert(self._h, int(rid), arr.ctypes.data if arr.size else None,
                                      int(arr.size)), "xattn_cht_insert")

    def best(self):
        rid, miss = ctypes.c_int64(0), ctypes.c_int64(0)
        _check(lib().xattn_cht_best(self._h, ctypes.byref(rid), ctypes.byref(miss)), "xattn_cht_best")
        return int(rid.value), int(miss.value)

    def admit(self, rid: int) -> None:
        _check(lib().xattn_cht_admit(self._h, int(rid)), "xattn_cht_admit")

    def complete(self, rid: int) -> None:
        _check(lib().xattn_cht_complete(self._h, int(rid)), "xattn_cht_complete")

    def form_batch(self, max_batch: int, max_missing: int):
        out = np.zeros(max(int(max_batch), 1), dtype=np.int64)
        n = ctypes.c_int32(0)
        _check(lib().xattn_cht_form_batch(self._h, int(max_batch), int(max_missing), out.ctypes.data,
                                          ctypes.byref(n)), "xattn_cht_form_batch")
        return [int(x) for x in out[:n.value]]

    def close(self):
        if self._h is not None and self._h.value:
            lib().xattn_cht_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def beam_topk(beam_score, logprob, token, n_out, parent, token_out, score_out, stream=None):
    """beam_score [R][BW], logprob / token [R][BW][K] -> parent / token_out / score_out [R][n_out]."""
    R, BW, K = (int(x) for x in logprob.shape)
    _check(lib().xattn_beam_topk(R, BW, K, int(n_out), _ptr(beam_score), _ptr(logprob), _ptr(token),
                                 _ptr(parent), _ptr(token_out), _ptr(score_out), _stream(stream)),
           "xattn_beam_topk")


def layer_step(dims, *, q, k_shared, v_shared, prefix_off, prefix_len, k_pool, v_pool, table_out,
               unshared_len, o, lse=None, workspace=None, workspace_bytes=0, k_new=None, v_new=None,
               parent=None, slot_base=None, active=None, table_in=None, decode_begin=None,
               decode_end=None) -> LayerStep:
    """Fill one xattn_layer_step from tensors (events: objects whose
    `cuda_event` is a hipEvent_t handle, or None).

    The returned object keeps every tensor and event it points to alive; a
    StepGraph keeps its LayerSteps, so a captured graph never refers to memory
    that was freed (and possibly handed to another tensor) behind it."""
    ev = lambda e: None if e is None else e.cuda_event
    st = LayerStep(dims, _ptr(k_new), _ptr(v_new), _ptr(parent), _ptr(slot_base), _ptr(active),
                   _ptr(table_in), _ptr(table_out), _ptr(unshared_len), _ptr(q), _ptr(k_shared),
                   _ptr(v_shared), _ptr(prefix_off), _ptr(prefix_len), _ptr(k_pool), _ptr(v_pool),
                   _ptr(o), _ptr(lse), _ptr(workspace), int(workspace_bytes), ev(decode_begin),
                   ev(decode_end))
    st.keep_alive = [x for x in (k_new, v_new, parent, slot_base, active, table_in, table_out,
                                 unshared_len, q, k_shared, v_shared, prefix_off, prefix_len, k_pool,
                                 v_pool, o, lse, workspace, decode_begin, decode_end)
                     if x is not None and not isinstance(x, int)]
    return st


def beam_select(beam_score, logprob, token, n_out, parent, token_out, score_out) -> BeamSelect:
    """Fill an xattn_beam_select from tensors (kept alive by the result)."""
    R, BW, K = (int(x) for x in logprob.shape)
    sel = BeamSelect(R, BW, K, int(n_out), _ptr(beam_score), _ptr(logprob), _ptr(token),
                     _ptr(parent), _ptr(token_out), _ptr(score_out))
    sel.keep_alive = [beam_score, logprob, token, parent, token_out, score_out]
    return sel


class StepGraph:
    """A captured multi-layer decode step (xattn_step_graph_*)."""

    def __init__(self, steps, select=None):
        # the LayerSteps' (and BeamSelect's) keep_alive lists pin the graph's buffers
        self._steps = list(steps)
        self._select = select
        arr = (LayerStep * max(len(steps), 1))(*steps)
        h = ctypes.c_void_p(None)
        _check(lib().xattn_step_graph_create(ctypes.byref(select) if select is not None else None,
                                             arr, len(steps), ctypes.byref(h)),
               "xattn_step_graph_create")
        self._h = h

    def launch(self, stream=None):
        _check(lib().xattn_step_graph_launch(self._h, _stream(stream)), "xattn_step_graph_launch")

    def close(self):
        if self._h is not None and self._h.value:
            _check(lib().xattn_step_graph_destroy(self._h), "xattn_step_graph_destroy")
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
