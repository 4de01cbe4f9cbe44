"""HIP path vs the fp64 oracle, through the C-ABI (needs an MI355X).

Inputs are seeded; the oracle consumes the same values the device is given.
Sizes here let the oracle finish in seconds while spanning several key tiles,
several row tiles and ragged tails; the full benchmark-shaped workloads are
checked on sampled rows in test_gpu_configs.py.
"""
import zlib

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from generative_recommendation_beam_amd import device as dv
from generative_recommendation_beam_amd import xattn
from generative_recommendation_beam_amd.inputs import make_workload
from oracle import attention as oa
from oracle import append as oapp
from parity import compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    xattn.lib()


def _np(t):
    return t.detach().cpu().numpy()


def run_decode(w, **kw):
    d = dv.upload(w, **kw)
    dv.build_cache(d)
    o, lse, ws, nb = dv.alloc_outputs(d, 2)
    dv.decode(d, o, lse, ws, nb)
    torch.cuda.synchronize()
    return d, _np(o)[:d.rows].reshape(w.N_b, w.Hq, w.D), _np(lse)[:d.rows].reshape(w.N_b, w.Hq)


CASES = {
    # name: make_workload kwargs
    "ragged_small_bf16": dict(R=3, B=5, Hq=8, Hkv=2, D=128, prefix_len=[150, 0, 67], unshared_len=[3, 1, 2], T_max=4),
    "mfma_multi_tile": dict(R=2, B=40, Hq=8, Hkv=2, D=128, prefix_len=[700, 333], unshared_len=[4, 2]),
    "d64_bf16": dict(R=2, B=24, Hq=4, Hkv=1, D=64, prefix_len=[257, 130], unshared_len=[2, 3]),
    "g8_bf16": dict(R=2, B=16, Hq=16, Hkv=2, D=128, prefix_len=[520, 64], unshared_len=[5, 1]),
    # four query heads per kv head, at most three generated tokens: with four
    # key groups the tokens go through one matrix-core block (lengths 0..3,
    # prompts of 0, 1 and several 128-key steps)
    "tb_mix_bf16": dict(R=4, B=30, Hq=8, Hkv=2, D=128, prefix_len=[600, 70, 0, 129], unshared_len=[3, 1, 2, 0]),
    "g16_bf16": dict(R=2, B=6, Hq=32, Hkv=2, D=128, prefix_len=[450, 130], unshared_len=[3, 2]),
    "g1_bf16": dict(R=2, B=20, Hq=2, Hkv=2, D=128, prefix_len=[99, 200], unshared_len=[1, 3]),
    "g6_bf16": dict(R=1, B=9, Hq=12, Hkv=2, D=128, prefix_len=[131], unshared_len=[2]),
    "b1_decode_bf16": dict(R=5, B=1, Hq=8, Hkv=2, D=128, prefix_len=[300, 64, 1, 0, 500], unshared_len=[3, 0, 2, 4, 1], T_max=5),
    "no_prefix_bf16": dict(R=2, B=8, Hq=8, Hkv=2, D=128, prefix_len=[0, 0], unshared_len=[3, 2]),
    "no_gen_bf16": dict(R=2, B=8, Hq=8, Hkv=2, D=128, prefix_len=[200, 90], unshared_len=[0, 0], T_max=2),
    "long_gen_bf16": dict(R=2, B=4, Hq=8, Hkv=2, D=128, prefix_len=[300, 100], unshared_len=[70, 45]),
    # generated tails longer than 16 tokens go to the vector kernel: every
    # query-head grouping (1, 2, 4 of 4, 6 of 8, 8) and head dim 64 in bf16
    "long_gen_d64_bf16": dict(R=2, B=3, Hq=4, Hkv=1, D=64, prefix_len=[130, 64], unshared_len=[40, 17]),
    "long_gen_g1_bf16": dict(R=2, B=4, Hq=2, Hkv=2, D=128, prefix_len=[99, 0], unshared_len=[30, 20]),
    "long_gen_g2_bf16": dict(R=1, B=5, Hq=4, Hkv=2, D=128, prefix_len=[300], unshared_len=[21]),
    "long_gen_g6_bf16": dict(R=2, B=2, Hq=12, Hkv=2, D=128, prefix_len=[64, 131], unshared_len=[19, 33]),
    "long_gen_g8_bf16": dict(R=1, B=4, Hq=16, Hkv=2, D=128, prefix_len=[200], unshared_len=[25]),
    "f32_small": dict(R=2, B=4, Hq=4, Hkv=1, D=64, prefix_len=[256, 100], unshared_len=[2, 3], dtype="f32"),
    "f32_d128": dict(R=1, B=3, Hq=8, Hkv=2, D=128, prefix_len=[190], unshared_len=[2], dtype="f32"),
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("std", [1.0, 0.3])
def test_decode_matches_oracle(name, std):
    kw = dict(CASES[name])
    w = make_workload(name, seed_key=(300, zlib.crc32(name.encode()) % 1000, int(std * 10)), qkv_std=std,
                      parent_dist="uniform", **kw)
    d, o, lse = run_decode(w)
    O, L = oa.attention(w)
    compare(o, O, lse, L, w.dtype, f"decode {name} std={std}")


@pytest.mark.parametrize("splits", [(1, 0), (2, 0), (3, 0), (5, 0), (1, 1), (2, 3), (4, 2)])
def test_decode_forced_splits(splits):
    ps, us = splits
    w = make_workload("splits", R=2, B=12, Hq=8, Hkv=2, D=128, prefix_len=[640, 200],
                      unshared_len=[6, 3], seed_key=(301, ps, us), parent_dist="zipf")
    d, o, lse = run_decode(w, prefix_splits=ps, unshared_splits=us)
    plan = xattn.get_plan(d.dims, 2)
    assert plan["prefix_splits"] >= 1
    O, L = oa.attention(w)
    compare(o, O, lse, L, "bf16", f"decode splits={splits} plan={plan}")


@pytest.mark.parametrize("shape,ps", [
    # 8 head-group query rows, 8 splits merged in one workgroup; the shorter
    # prompt leaves most of its splits empty
    (dict(R=2, B=3, Hq=8, Hkv=1, D=128, prefix_len=[500, 40], unshared_len=[3, 1]), 8),
    # 3 query heads per kv head (one masked group of 8), an empty prompt, no tail
    (dict(R=3, B=2, Hq=3, Hkv=1, D=64, prefix_len=[300, 0, 129], unshared_len=[2, 2, 0], T_max=3), 5),
    # one query head per kv head; 9 splits: partials and a Merge launch instead
    (dict(R=2, B=5, Hq=2, Hkv=2, D=64, prefix_len=[1100, 333], unshared_len=[1, 4]), 9),
])
def test_f32_vector_splits(shape, ps):
    w = make_workload("f32_splits", dtype="f32", seed_key=(305, ps), parent_dist="uniform", **shape)
    d, o, lse = run_decode(w, prefix_splits=ps)
    plan = xattn.get_plan(d.dims, 2)
    assert plan["mfma"] == 0 and plan["prefix_splits"] == ps and (plan["partials"] == 0) == (ps <= 8), plan
    O, L = oa.attention(w)
    compare(o, O, lse, L, "f32", f"f32 vector splits={ps} plan={plan}")


KG_CASES = ["ragged_small_bf16", "mfma_multi_tile", "d64_bf16", "g8_bf16", "g16_bf16", "g6_bf16", "no_prefix_bf16",
            "tb_mix_bf16",
            "no_gen_bf16", "long_gen_bf16"]


KG_PLANS = [(64, 0, 2, 2), (128, 0, 2, 2), (32, 0, 2, 2), (64, 3, 2, 2),
            (64, 0, 4, 2), (128, 0, 4, 2), (32, 0, 4, 2), (64, 3, 4, 2),
            (64, 0, 2, 4), (32, 0, 2, 4), (64, 3, 2, 4)]
# Four key groups exist for head dim 128 only; the ABI's rejection of the
# others (XATTN_ERR_UNSUPPORTED) is checked in test_abi.py.
KG_RUNS = [(n,) + p for n in KG_CASES for p in KG_PLANS if p[3] != 4 or CASES[n]["D"] == 128]


@pytest.mark.parametrize("name,rows,ps,stages,kg", KG_RUNS)
def test_decode_key_groups(name, rows, ps, stages, kg):
    """Wave groups per workgroup split the keys of the same rows: two groups
    on alternate 64-key tiles (2 stages) or on the two halves of every tile
    (4 stages); four groups on the halves of two tiles a step. Prompts here
    end inside any group's share, or leave some groups none."""
    w = make_workload(name, seed_key=(305, rows, ps, kg, zlib.crc32(name.encode()) % 1000), **CASES[name])
    d, o, lse = run_decode(w, rows_per_block=rows, key_groups=kg, prefix_splits=ps, pipeline_stages=stages)
    plan = xattn.get_plan(d.dims, 2)
    assert plan["mfma"] == 1 and plan["key_groups"] == kg and plan["rows_per_block"] == rows
    assert plan["pipeline_stages"] == stages
    O, L = oa.attention(w)
    compare(o, O, lse, L, w.dtype, f"decode key groups {name} plan={plan}")


@pytest.mark.parametrize("rows,kg", [(64, 4), (32, 4), (64, 2)])
def test_decode_late_score_jump(rows, kg):
    """Keys 40 and 41 of a 300-key prompt score ~130 log2 units above every
    other key, for every query row, and arrive after other keys of the same
    group have set its running maximum: the accumulated output must be
    rescaled by about 2^-127 without losing the later keys' weights."""
    w = make_workload("jump", R=1, B=16, Hq=8, Hkv=2, D=128, prefix_len=[300], unshared_len=[2],
                      seed_key=(312, rows, kg))
    w.q[:] = 0x3F80                      # bf16 1.0: a query row's score is its key's row sum
    w.k_shared[:, 40, :] = 0x4100        # bf16 8.0: score 1024 * scale
    w.k_shared[:, 41, :] = 0x4100
    w.k_shared[:, 41, :8] = 0x40E0       # bf16 7.0: score 1016 * scale, a visible second weight
    d, o, lse = run_decode(w, rows_per_block=rows, key_groups=kg)
    plan = xattn.get_plan(d.dims, 2)
    assert plan["key_groups"] == kg and plan["rows_per_block"] == rows
    O, L = oa.attention(w)
    compare(o, O, lse, L, "bf16", f"late score jump plan={plan}")


@pytest.mark.parametrize("stage", ["unshared", "decode"])
def test_vector_late_score_jump_generated(stage):
    """Generated token 40 of a 70-token tail scores ~130 log2 units above
    every other key, for every query row. The vector kernel's four key slots
    take keys 4 apart, so only one slot sees it, after that slot's running
    maximum was set by ten ordinary keys: that slot must rescale its
    accumulated output by about 2^-127 (the lazy rescale's branch with a
    finite maximum), and the slot combine must then give the other slots'
    far smaller weights their due."""
    w = make_workload("vjump", R=2, B=3, Hq=8, Hkv=2, D=128, prefix_len=[0, 150], unshared_len=[70, 70],
                      seed_key=(313, 0))
    w.q[:] = 0x3F80                    # bf16 1.0: a row's score is its key's row sum
    w.k_new[40] = 0x4100               # bf16 8.0: score 1024 * scale for token 40 of every beam
    w.k_new[40, :, :, :8] = 0x40E0     # slightly lower on a few elements: still the maximum by far
    d = dv.upload(w)
    dv.build_cache(d)
    if stage == "unshared":
        o, lse, ws, nb = dv.alloc_outputs(d, 1)
        dv.unshared_stage(d, o, lse, ws, nb)
        O, L = oa.attention(w, include_prefix=False)
    else:
        o, lse, ws, nb = dv.alloc_outputs(d, 2)
        dv.decode(d, o, lse, ws, nb)
        O, L = oa.attention(w)
    torch.cuda.synchronize()
    compare(_np(o)[:d.rows].reshape(O.shape), O, _np(lse)[:d.rows].reshape(L.shape), L, "bf16",
            f"vector late score jump ({stage})")


def test_vector_late_score_jump_f32_prompt():
    """fp32 prompts run on the vector kernel: prompt key 40 of 300 (one key
    slot) jumps ~130 log2 units above the rest after that slot has seen ten
    keys; an fp32 generated tail follows."""
    w = make_workload("vjump32", R=1, B=4, Hq=4, Hkv=1, D=64, prefix_len=[300], unshared_len=[3], dtype="f32",
                      seed_key=(314, 0))
    w.q[:] = 1.0
    w.k_shared[:, 40, :] = 16.0        # score 1024 * scale
    d, o, lse = run_decode(w)
    plan = xattn.get_plan(d.dims, 2)
    assert plan["mfma"] == 0, plan
    O, L = oa.attention(w)
    compare(o, O, lse, L, "f32", "fp32 vector late score jump")


@pytest.mark.parametrize("name", ["ragged_small_bf16", "mfma_multi_tile", "b1_decode_bf16", "f32_small"])
@pytest.mark.parametrize("ps", [0, 3])
@pytest.mark.parametrize("kg", [0, 2])
def test_shared_stage_matches_oracle(name, ps, kg):
    """Shared stage alone; single-beam bf16 prompts run on the MFMA kernel
    too (a 32-row tile), with and without key groups and prompt splits.
    fp32 prompts run on the vector kernel, which takes no key groups: the
    forced value is ignored there."""
    w = make_workload(name, seed_key=(302, ps), **CASES[name])
    d = dv.upload(w, prefix_splits=ps, key_groups=kg)
    plan = xattn.get_plan(d.dims, 0)
    if CASES[name].get("dtype") == "f32":
        assert plan["mfma"] == 0 and plan["key_groups"] == 0, plan
    else:
        assert plan["mfma"] == 1 and plan["key_groups"] == (kg or plan["key_groups"]), plan
    o, lse, ws, nb = dv.alloc_outputs(d, 0)
    dv.shared_stage(d, o, lse, ws, nb)
    torch.cuda.synchronize()
    O, L = oa.attention(w, include_generated=False)
    compare(_np(o)[:d.rows].reshape(O.shape), O, _np(lse)[:d.rows].reshape(L.shape), L, w.dtype,
            f"shared {name}")


@pytest.mark.parametrize("name", ["ragged_small_bf16", "long_gen_bf16", "b1_decode_bf16", "f32_small",
                                  "d64_bf16", "g1_bf16", "g6_bf16", "g8_bf16", "g16_bf16",
                                  "long_gen_d64_bf16", "long_gen_g1_bf16", "long_gen_g2_bf16",
                                  "long_gen_g6_bf16", "long_gen_g8_bf16"])
@pytest.mark.parametrize("us", [0, 4])
def test_unshared_stage_matches_oracle(name, us):
    w = make_workload(name, seed_key=(303, us), **CASES[name])
    d = dv.upload(w, unshared_splits=us)
    dv.build_cache(d)
    o, lse, ws, nb = dv.alloc_outputs(d, 1)
    dv.unshared_stage(d, o, lse, ws, nb)
    torch.cuda.synchronize()
    O, L = oa.attention(w, include_prefix=False)
    compare(_np(o)[:d.rows].reshape(O.shape), O, _np(lse)[:d.rows].reshape(L.shape), L, w.dtype,
            f"unshared {name}")


def test_merge_matches_oracle():
    rng = np.random.default_rng(7)
    rows, D = 1000, 128
    oa_ = rng.standard_normal((rows, D)).astype(np.float32)
    ob_ = rng.standard_normal((rows, D)).astype(np.float32)
    la = (rng.standard_normal(rows) * 5).astype(np.float32)
    lb = (rng.standard_normal(rows) * 5).astype(np.float32)
    la[::7] = -np.inf
    lb[::11] = -np.inf
    t = lambda a: torch.from_numpy(a).cuda()
    A, Bt, LA, LB = t(oa_), t(ob_), t(la), t(lb)
    out = torch.empty_like(A)
    lout = torch.empty_like(LA)
    xattn.merge(rows, D, A, LA, Bt, LB, out, lout)
    torch.cuda.synchronize()
    Om, Lm = oa.merge(oa_, la, ob_, lb)
    compare(_np(out), Om, _np(lout), Lm, "f32", "merge")
    # in place: o_out aliases o_a and lse_out aliases lse_a
    xattn.merge(rows, D, A, LA, Bt, LB, A, LA)
    torch.cuda.synchronize()
    compare(_np(A), Om, _np(LA), Lm, "f32", "merge in place")


def test_merge_of_stages_equals_decode():
    w = make_workload("stages", R=2, B=16, Hq=8, Hkv=2, D=128, prefix_len=[500, 77],
                      unshared_len=[3, 2], seed_key=(304, 0))
    d = dv.upload(w)
    dv.build_cache(d)
    os_, ls_, ws0, n0 = dv.alloc_outputs(d, 0)
    ou_, lu_, ws1, n1 = dv.alloc_outputs(d, 1)
    dv.shared_stage(d, os_, ls_, ws0, n0)
    dv.unshared_stage(d, ou_, lu_, ws1, n1)
    xattn.merge(d.rows, w.D, os_, ls_, ou_, lu_, os_, ls_)
    torch.cuda.synchronize()
    O, L = oa.attention(w)
    compare(_np(os_)[:d.rows].reshape(O.shape), O, _np(ls_)[:d.rows].reshape(L.shape), L, "bf16",
            "shared+unshared+merge")


# ---------------------------------------------------------------- append

def _oracle_append(w, inplace=True):
    kpool = np.zeros((w.num_slots, w.Hkv, w.D), dtype=w.k_new.dtype)
    vpool = np.zeros_like(kpool)
    table = np.full((w.N_b, w.T_max), -1, dtype=np.int64)
    ulen = np.zeros(w.R, dtype=np.int64)
    for t in range(w.T_steps):
        tout = table if inplace else table.copy()
        oapp.cache_append(B=w.B, k_new=w.k_new[t], v_new=w.v_new[t], parent=w.parents[t],
                          slot_base=w.slot_base, active=w.active(t), k_pool=kpool, v_pool=vpool,
                          table_in=table, table_out=tout, unshared_len=ulen)
        table = tout
    return kpool, vpool, table, ulen


@pytest.mark.parametrize("parent", ["uniform", "zipf", "identity", "zero", "reverse"])
@pytest.mark.parametrize("inplace", [True, False])
def test_append_bit_exact(parent, inplace):
    w = make_workload("app", R=3, B=37, Hq=4, Hkv=2, D=64, prefix_len=1,
                      unshared_len=[6, 3, 0], seed_key=(305, 0),
                      parent_dist="uniform" if parent in ("zero", "reverse") else parent, T_max=7)
    if parent in ("zero", "reverse"):
        for t in range(1, w.T_steps):
            for r in range(w.R):
                bb = np.arange(w.B)
                w.parents[t, r * w.B:(r + 1) * w.B] = 0 * bb if parent == "zero" else bb[::-1]
    d = dv.upload(w)
    cur = d.table
    for t in range(w.T_steps):
        if inplace:
            dv.append_step(d, t)
        else:
            nxt = cur.clone()          # ping-pong: the new table starts as a copy
            dv.append_step(d, t, table_in=cur, table_out=nxt)
            cur = nxt
    torch.cuda.synchronize()
    kpool, vpool, table, ulen = _oracle_append(w, inplace)
    assert np.array_equal(_np(d.unshared_len)[:w.R], ulen)
    assert np.array_equal(_np(cur if not inplace else d.table).astype(np.int64), table)
    kp = _np(d.k_pool.view(torch.int16)).view(np.uint16) if w.dtype == "bf16" else _np(d.k_pool)
    vp = _np(d.v_pool.view(torch.int16)).view(np.uint16) if w.dtype == "bf16" else _np(d.v_pool)
    assert np.array_equal(kp, kpool) and np.array_equal(vp, vpool)


def test_append_large_beam_column_chunks():
    """B large enough that one request's table needs several column chunks."""
    w = make_workload("appB", R=2, B=3000, Hq=1, Hkv=1, D=64, prefix_len=1, unshared_len=[5, 4],
                      seed_key=(306, 0), parent_dist="zipf", T_max=5)
    d = dv.upload(w)
    dv.build_cache(d)
    torch.cuda.synchronize()
    kpool, vpool, table, ulen = _oracle_append(w)
    assert np.array_equal(_np(d.table).astype(np.int64), table)
    assert np.array_equal(_np(d.unshared_len)[:w.R], ulen)
    kp = _np(d.k_pool.view(torch.int16)).view(np.uint16)
    vp = _np(d.v_pool.view(torch.int16)).view(np.uint16)
    assert np.array_equal(kp, kpool) and np.array_equal(vp, vpool)


def test_append_long_rows_column_chunks():
    """Small B with long rows: each request's table spans two column chunks,
    the second one ragged, and t crosses the chunk boundary during the run."""
    w = make_workload("appL", R=2, B=5, Hq=2, Hkv=1, D=64, prefix_len=1, unshared_len=[450, 300],
                      seed_key=(311, 0), parent_dist="uniform", T_max=450)
    d = dv.upload(w)
    dv.build_cache(d)
    torch.cuda.synchronize()
    kpool, vpool, table, ulen = _oracle_append(w)
    assert np.array_equal(_np(d.table).astype(np.int64), table)
    assert np.array_equal(_np(d.unshared_len)[:w.R], ulen)
    kp = _np(d.k_pool.view(torch.int16)).view(np.uint16)
    vp = _np(d.v_pool.view(torch.int16)).view(np.uint16)
    assert np.array_equal(kp, kpool) and np.array_equal(vp, vpool)


def test_append_on_full_row_changes_nothing():
    """An append on requests whose rows are full writes nothing and leaves the
    lengths as they are (every workgroup still arrives once)."""
    w = make_workload("full", R=3, B=24, Hq=4, Hkv=2, D=128, prefix_len=1, unshared_len=[4, 4, 2],
                      seed_key=(310, 0), T_max=4)
    d = dv.upload(w)
    dv.build_cache(d)
    torch.cuda.synchronize()
    before = [_np(x).copy() for x in (d.unshared_len, d.table, d.k_pool.view(torch.int16), d.v_pool.view(torch.int16))]
    active = torch.tensor([1, 1, 0], dtype=torch.uint8, device=d.q.device)
    xattn.cache_append(d.dims, d.k_new[0], d.v_new[0], d.parents[1], d.slot_base, active, d.k_pool, d.v_pool,
                       d.table, d.table, d.unshared_len)
    torch.cuda.synchronize()
    after = [_np(x) for x in (d.unshared_len, d.table, d.k_pool.view(torch.int16), d.v_pool.view(torch.int16))]
    for b, a in zip(before, after):
        assert np.array_equal(b, a)
    assert list(after[0][:3]) == [4, 4, 2]


def test_decode_identical_histories_bitwise():
    w = make_workload("ih", R=1, B=32, Hq=8, Hkv=2, D=128, prefix_len=300, unshared_len=3,
                      seed_key=(307, 0))
    n1, n2 = 3, 17
    w.q[n2] = w.q[n1]
    for t in range(w.T_steps):
        w.parents[t, n2] = w.parents[t, n1]
        w.k_new[t, n2] = w.k_new[t, n1]
        w.v_new[t, n2] = w.v_new[t, n1]
    d, o, lse = run_decode(w)
    assert np.array_equal(o[n1], o[n2]) and np.array_equal(lse[n1], lse[n2])


def test_workspace_reuse_across_split_counts():
    """One zero-initialised workspace serves repeated calls with different
    split counts: the in-kernel split counters return to zero after each."""
    w = make_workload("reuse", R=2, B=32, Hq=8, Hkv=2, D=128, prefix_len=[900, 700],
                      unshared_len=[3, 2], seed_key=(309, 0))
    O, L = oa.attention(w)
    d = dv.upload(w, prefix_splits=7)
    dv.build_cache(d)
    _, _, ws, nb = dv.alloc_outputs(d, 2)
    for ps in (7, 3, 7, 2, 5, 5):
        d.dims.prefix_splits = ps
        o, lse, _, nb2 = dv.alloc_outputs(d, 2)
        assert nb2 <= ws.numel()
        dv.decode(d, o, lse, ws, ws.numel())
        torch.cuda.synchronize()
        compare(_np(o)[:d.rows].reshape(O.shape), O, _np(lse)[:d.rows].reshape(L.shape), L, "bf16",
                f"reuse ps={ps}")


def test_decode_deterministic():
    w = make_workload("det", R=2, B=64, Hq=8, Hkv=2, D=128, prefix_len=900, unshared_len=3,
                      seed_key=(308, 0))
    d = dv.upload(w, prefix_splits=3)
    dv.build_cache(d)
    o, lse, ws, nb = dv.alloc_outputs(d, 2)
    dv.decode(d, o, lse, ws, nb)
    o1 = o.clone()
    dv.decode(d, o, lse, ws, nb)
    torch.cuda.synchronize()
    assert torch.equal(o, o1)
