"""xattn_append_decode: the cache append folded into the decode launch.

The fused call must give, bit for bit, what xattn_cache_append followed by
xattn_decode gives from the same state (outputs, pools, output table,
lengths), and the attention must match the oracle on the final cache. Plans
that cannot fold (long generated tails, prompt splits) take the two-call
path inside the same entry point and are checked the same way.
"""
import zlib

import numpy as np
import pytest
import torch

from generative_recommendation_beam_amd import device as dv
from generative_recommendation_beam_amd import xattn
from generative_recommendation_beam_amd.inputs import make_workload
from oracle import attention as oa
from parity import compare

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().cpu().numpy()


ONE = dict(prefix_splits=1)  # one prompt range: the append folds into the decode launch
CASES = {
    # name: (make_workload kwargs, upload overrides, folds)
    "gr_kg4": (dict(R=3, B=32, Hq=8, Hkv=2, D=128, prefix_len=[600, 300, 1000], unshared_len=[3, 3, 3]),
               dict(ONE, key_groups=4, rows_per_block=64), True),
    "kg1_rows128": (dict(R=2, B=64, Hq=8, Hkv=2, D=128, prefix_len=[700, 333], unshared_len=[4, 2]),
                    dict(ONE, key_groups=1, rows_per_block=128), True),
    "kg2_rows64": (dict(R=2, B=40, Hq=8, Hkv=2, D=128, prefix_len=[513, 129], unshared_len=[5, 5]),
                   dict(ONE, key_groups=2, rows_per_block=64), True),
    "kg4_g8_short": (dict(R=2, B=12, Hq=16, Hkv=2, D=128, prefix_len=[400, 150], unshared_len=[2, 1]),
                     dict(ONE, key_groups=4, rows_per_block=64), True),
    "kg4_inactive_mix": (dict(R=4, B=30, Hq=8, Hkv=2, D=128, prefix_len=[600, 70, 0, 333],
                              unshared_len=[3, 1, 0, 2], T_max=3), dict(ONE, key_groups=4, rows_per_block=64), True),
    "kg4_rows32": (dict(R=2, B=24, Hq=8, Hkv=2, D=128, prefix_len=[300, 77], unshared_len=[2, 3]),
                   dict(ONE, key_groups=4, rows_per_block=32), True),
    "kg1_rows64_nw2": (dict(R=2, B=30, Hq=8, Hkv=2, D=128, prefix_len=[410, 64], unshared_len=[6, 2]),
                       dict(ONE, key_groups=1, rows_per_block=64), True),
    "kg1_stages4": (dict(R=2, B=32, Hq=8, Hkv=2, D=128, prefix_len=[530, 200], unshared_len=[3, 3]),
                    dict(ONE, key_groups=1, rows_per_block=128, pipeline_stages=4), True),
    "g3_straddle": (dict(R=2, B=30, Hq=6, Hkv=2, D=128, prefix_len=[250, 190], unshared_len=[3, 2]),
                    dict(ONE, key_groups=1, rows_per_block=64), True),
    "g3_straddle_kg4": (dict(R=2, B=30, Hq=6, Hkv=2, D=128, prefix_len=[250, 190], unshared_len=[3, 2]),
                        dict(ONE, key_groups=4, rows_per_block=64), True),
    "inactive_mix": (dict(R=4, B=16, Hq=8, Hkv=2, D=128, prefix_len=[200, 0, 90, 333],
                          unshared_len=[4, 1, 0, 2], T_max=6), ONE, True),
    "full_rows": (dict(R=2, B=16, Hq=8, Hkv=2, D=128, prefix_len=[150, 260], unshared_len=[4, 2], T_max=4),
                  ONE, True),
    "first_step": (dict(R=2, B=16, Hq=8, Hkv=2, D=128, prefix_len=[180, 90], unshared_len=[1, 1]), ONE, True),
    "no_prompt": (dict(R=2, B=16, Hq=8, Hkv=2, D=128, prefix_len=[0, 0], unshared_len=[3, 2]), ONE, True),
    "d64": (dict(R=2, B=24, Hq=4, Hkv=1, D=64, prefix_len=[257, 130], unshared_len=[2, 3]), ONE, True),
    "auto_plan": (dict(R=3, B=32, Hq=8, Hkv=2, D=128, prefix_len=[600, 300, 1000], unshared_len=[3, 3, 3]),
                  {}, False),
    "fallback_long": (dict(R=2, B=4, Hq=8, Hkv=2, D=128, prefix_len=[300, 100], unshared_len=[40, 25]), ONE,
                      False),
    # long generated tails: the append folds into the prompt pass (split 0's
    # workgroups), then the Non-Shared pass and the Merge
    "long_splits": (dict(R=2, B=4, Hq=8, Hkv=2, D=128, prefix_len=[1500, 600], unshared_len=[40, 20]),
                    dict(prefix_splits=3), False),
    "long_full_rows": (dict(R=2, B=4, Hq=8, Hkv=2, D=128, prefix_len=[150, 260], unshared_len=[20, 18],
                            T_max=20), ONE, False),
    "long_no_prompt": (dict(R=2, B=3, Hq=4, Hkv=1, D=64, prefix_len=[0, 130], unshared_len=[30, 25]), ONE,
                       False),
    # the Non-Shared pass's splits as the waves of one workgroup folding the
    # prompt partials in: more query heads than splits, fewer, and eight
    "long_fold_3splits": (dict(R=2, B=3, Hq=8, Hkv=2, D=128, prefix_len=[900, 200], unshared_len=[70, 41]),
                          dict(unshared_splits=3), False),
    "long_fold_8splits_g8": (dict(R=1, B=4, Hq=16, Hkv=2, D=128, prefix_len=[700], unshared_len=[90]),
                             dict(unshared_splits=8, prefix_splits=2), False),
    "long_fold_2splits_d64": (dict(R=2, B=2, Hq=4, Hkv=1, D=64, prefix_len=[300, 0], unshared_len=[33, 20]),
                              dict(unshared_splits=2), False),
    # tails of 64 tokens or more per Non-Shared split: the vector kernel's
    # batched updates, with the four heads of G = 4 spread over a key slot's
    # lanes (head dims 128 and 64) and the plain batches for G = 8, 6
    # (one masked head group), 2 and 1; partial last batches throughout
    "batch_g4": (dict(R=2, B=3, Hq=8, Hkv=2, D=128, prefix_len=[400, 130], unshared_len=[150, 77]), {}, False),
    "batch_g4_d64": (dict(R=2, B=2, Hq=4, Hkv=1, D=64, prefix_len=[300, 0], unshared_len=[100, 65]), {}, False),
    "batch_g8": (dict(R=1, B=4, Hq=16, Hkv=2, D=128, prefix_len=[500], unshared_len=[130]), {}, False),
    "batch_g6": (dict(R=1, B=3, Hq=12, Hkv=2, D=128, prefix_len=[256], unshared_len=[90]), {}, False),
    "batch_g2": (dict(R=2, B=3, Hq=4, Hkv=2, D=128, prefix_len=[200, 64], unshared_len=[96, 70]), {}, False),
    "batch_g1": (dict(R=1, B=4, Hq=2, Hkv=2, D=64, prefix_len=[128], unshared_len=[80]), {}, False),
    "fallback_splits": (dict(R=2, B=12, Hq=8, Hkv=2, D=128, prefix_len=[640, 200], unshared_len=[3, 2]),
                        dict(prefix_splits=3), False),
    "fallback_f32": (dict(R=2, B=4, Hq=4, Hkv=1, D=64, prefix_len=[256, 100], unshared_len=[2, 3],
                          dtype="f32"), {}, False),
    # single-beam prompts on the matrix cores: a beam's few query rows in one
    # 32-row tile (four key groups from 512-key prompts at head dim 128)
    "one_beam_kg4": (dict(R=3, B=1, Hq=8, Hkv=2, D=128, prefix_len=[700, 512, 90], unshared_len=[3, 2, 1]),
                     ONE, True),
    "two_beams_g8": (dict(R=2, B=2, Hq=16, Hkv=2, D=128, prefix_len=[600, 300], unshared_len=[3, 1]), ONE, True),
    "one_beam_d64": (dict(R=2, B=1, Hq=4, Hkv=1, D=64, prefix_len=[520, 33], unshared_len=[2, 2]), ONE, True),
    "one_beam_splits": (dict(R=2, B=1, Hq=8, Hkv=2, D=128, prefix_len=[1500, 700], unshared_len=[3, 2]), {},
                        False),
}


def _state(d, table_out):
    return dict(k=d.k_pool.clone(), v=d.v_pool.clone(), tout=table_out.clone(), ulen=d.unshared_len.clone())


@pytest.mark.parametrize("name", sorted(CASES))
def test_append_decode_matches_two_calls_and_oracle(name):
    kw, up, folds = CASES[name]
    w = make_workload(name, seed_key=(320, zlib.crc32(name.encode()) % 1000), parent_dist="uniform", **kw)
    d = dv.upload(w, **up)
    plan = xattn.get_plan(d.dims, 2)
    assert (plan["mfma"] == 1 and plan["partials"] == 0 and w.T_max <= 16) == folds, plan
    # a folded append needs only the arrival counters
    assert (xattn.workspace_size(d.dims, 3) == 256 * -(-w.R * w.Hkv * 4 // 256)) == folds
    table_in, table_out, t = dv.prepare_step(d)
    assert t is not None
    ref = _state(d, table_out)
    fus = _state(d, table_out)
    o_r, lse_r, ws, nb = dv.alloc_outputs(d, 2)
    o_f, lse_f, ws3, nb3 = dv.alloc_outputs(d, 3)
    args = dict(q=d.q, k_shared=d.k_shared, v_shared=d.v_shared, prefix_off=d.prefix_off,
                prefix_len=d.prefix_len)
    xattn.cache_append(d.dims, d.k_new[t], d.v_new[t], d.parents[t], d.slot_base, d.active[t], ref["k"],
                       ref["v"], table_in, ref["tout"], ref["ulen"])
    xattn.decode(d.dims, d.q, d.k_shared, d.v_shared, d.prefix_off, d.prefix_len, ref["k"], ref["v"],
                 ref["tout"], ref["ulen"], o_r, lse_r, ws if nb else None, nb)
    xattn.append_decode(d.dims, k_new=d.k_new[t], v_new=d.v_new[t], parent=d.parents[t], slot_base=d.slot_base,
                        active=d.active[t], k_pool=fus["k"], v_pool=fus["v"], table_in=table_in,
                        table_out=fus["tout"], unshared_len=fus["ulen"], o=o_f, lse=lse_f,
                        workspace=ws3 if nb3 else None, workspace_bytes=nb3, **args)
    torch.cuda.synchronize()
    assert not ws3[:4 * w.R * w.Hkv].any()  # arrival (and split) counters back at zero
    torch.cuda.synchronize()
    rows = d.rows
    assert np.array_equal(_np(ref["ulen"]), _np(fus["ulen"]))
    assert np.array_equal(_np(ref["tout"]), _np(fus["tout"]))
    for k in ("k", "v"):
        assert torch.equal(ref[k].view(torch.int16) if ref[k].dtype == torch.bfloat16 else ref[k],
                           fus[k].view(torch.int16) if fus[k].dtype == torch.bfloat16 else fus[k])
    assert np.array_equal(_np(o_r)[:rows], _np(o_f)[:rows])
    assert np.array_equal(_np(lse_r)[:rows], _np(lse_f)[:rows])
    O, L = oa.attention(w)
    compare(_np(o_f)[:rows].reshape(O.shape), O, _np(lse_f)[:rows].reshape(L.shape), L, w.dtype,
            f"append_decode {name} plan={xattn.get_plan(d.dims, 2)}")


def test_append_decode_repeat_on_full_rows_changes_nothing():
    """A second fused call on rows that are now full: lengths, pools and the
    output table (copies of the input rows) stay as they are, and the
    attention is that of the full rows."""
    w = make_workload("full2", R=2, B=16, Hq=8, Hkv=2, D=128, prefix_len=[150, 260], unshared_len=[4, 4],
                      seed_key=(321, 0), parent_dist="uniform", T_max=4)
    d = dv.upload(w, **ONE)
    dv.build_cache(d)  # every row full
    torch.cuda.synchronize()
    before = dict(k=d.k_pool.clone(), v=d.v_pool.clone(), ulen=d.unshared_len.clone())
    tout = torch.full_like(d.table, -7)
    o, lse, ws, nb = dv.alloc_outputs(d, 3)
    t = w.T_steps - 1
    xattn.append_decode(d.dims, q=d.q, k_shared=d.k_shared, v_shared=d.v_shared, prefix_off=d.prefix_off,
                        prefix_len=d.prefix_len, k_new=d.k_new[t], v_new=d.v_new[t], parent=d.parents[t],
                        slot_base=d.slot_base, active=None, k_pool=d.k_pool, v_pool=d.v_pool,
                        table_in=d.table, table_out=tout, unshared_len=d.unshared_len, o=o, lse=lse,
                        workspace=ws if nb else None, workspace_bytes=nb)
    torch.cuda.synchronize()
    assert torch.equal(before["ulen"], d.unshared_len)
    assert torch.equal(before["k"].view(torch.int16), d.k_pool.view(torch.int16))
    assert torch.equal(before["v"].view(torch.int16), d.v_pool.view(torch.int16))
    assert torch.equal(tout, d.table)
    O, L = oa.attention(w)
    compare(_np(o)[:d.rows].reshape(O.shape), O, _np(lse)[:d.rows].reshape(L.shape), L, "bf16", "full rows")


def test_append_decode_rejects_in_place_tables():
    w = make_workload("inplace", R=1, B=4, Hq=4, Hkv=1, D=128, prefix_len=[64], unshared_len=[2],
                      seed_key=(322, 0))
    d = dv.upload(w)
    o, lse, ws, nb = dv.alloc_outputs(d, 3)
    with pytest.raises(RuntimeError):
        xattn.append_decode(d.dims, q=d.q, k_shared=d.k_shared, v_shared=d.v_shared, prefix_off=d.prefix_off,
                            prefix_len=d.prefix_len, k_new=d.k_new[0], v_new=d.v_new[0], parent=d.parents[0],
                            slot_base=d.slot_base, active=None, k_pool=d.k_pool, v_pool=d.v_pool,
                            table_in=d.table, table_out=d.table, unshared_len=d.unshared_len, o=o, lse=lse,
                            workspace=ws if nb else None, workspace_bytes=nb)


@pytest.mark.parametrize("shape", [
    # single-beam requests (one 32-row tile per (request, kv head)), and a
    # request of 16 beams x 4 heads (one 64-row tile), each with a long tail
    dict(R=4, B=1, Hq=8, Hkv=2, D=128, prefix_len=[700, 512, 90, 300], unshared_len=[3, 2, 1, 3]),
    dict(R=2, B=16, Hq=8, Hkv=2, D=128, prefix_len=[1100, 600], unshared_len=[40, 33]),
])
def test_disjoint_prompt_hint_changes_no_bit(shape):
    """prompts_disjoint only chooses the prompt loads' cache policy: the same
    call with the hint set (non-temporal loads where a workgroup alone reads
    its prompt) and cleared gives the same bits."""
    w = make_workload("hint", seed_key=(321, shape["B"]), parent_dist="uniform", **shape)
    outs = []
    for hint in (1, 0):
        d = dv.upload(w)
        assert d.dims.prompts_disjoint == 1  # distinct prompt ranges
        d.dims.prompts_disjoint = hint
        plan = xattn.get_plan(d.dims, 2)
        assert plan["mfma"] == 1 and plan["row_tiles"] == 1, plan
        dv.build_cache(d)
        o, lse, ws, nb = dv.alloc_outputs(d, 2)
        dv.decode(d, o, lse, ws, nb)
        torch.cuda.synchronize()
        outs.append((_np(o)[:d.rows].copy(), _np(lse)[:d.rows].copy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    O, L = oa.attention(w)
    compare(outs[0][0].reshape(O.shape), O, outs[0][1].reshape(L.shape), L, "bf16", "disjoint prompt hint")
