"""Reference semantics of the token-granular Non-Shared cache update.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py). Pure-Python loops, small
inputs only.

xGR page, section 2.1 xAttention: the Non-Shared cache is managed per token,
not per block, so a beam that branches needs no physical block copy; updates
happen in place through direct indices without read-before-write hazards.

Reading taken here (the page gives no allocator):
  * new beam b of request r at step t = unshared_len[r] is stored in pool slot
    slot_base[r] + t * B + b (a step-major slab per request);
  * its slot-table row becomes its parent's row over columns [0, t), then
    the new slot in column t; columns beyond t are not written;
  * all parent rows are read before any row is written, so an in-place update
    (table_out is table_in) equals an out-of-place one;
  * at t = 0 parents are ignored; inactive requests are left untouched;
  * unshared_len[r] is then incremented.
"""
from __future__ import annotations

import numpy as np


def cache_append(*, B, k_new, v_new, parent, slot_base, active, k_pool, v_pool,
                 table_in, table_out, unshared_len):
    """Apply one decode step's append. Arrays are numpy; k_pool, v_pool,
    table_out and unshared_len are updated and also returned.

    k_new, v_new: [N_b, H_kv, D]; parent: [N_b]; slot_base: [R];
    active: [R] or None; k_pool, v_pool: [num_slots, H_kv, D];
    table_in, table_out: [N_b, T_max] int32 (may be the same object);
    unshared_len: [R] int32.
    """
    R = len(slot_base)
    T_max = table_in.shape[1]
    old = [[int(x) for x in row] for row in table_in]   # every read happens first
    for r in range(R):
        if active is not None and not active[r]:
            continue
        t = int(unshared_len[r])
        if t >= T_max:
            raise ValueError("slot table row is full")
        for b in range(B):
            n = r * B + b
            if t > 0:
                p = r * B + int(parent[n])
                for j in range(t):
                    table_out[n, j] = old[p][j]
            slot = int(slot_base[r]) + t * B + b
            table_out[n, t] = slot
            k_pool[slot] = k_new[n]
            v_pool[slot] = v_new[n]
    for r in range(R):
        if active is None or active[r]:
            unshared_len[r] += 1
    return k_pool, v_pool, table_out, unshared_len
