"""The benchmark-shaped workloads at full size, through the C-ABI, in the
launch configuration bench.py times (automatic plan).

Coverage at full size:
  * outputs and lse start as NaN, so a row that no workgroup writes fails
    the all-finite check on the whole output;
  * the oracle recomputes one query row from every (request, kv head, row
    tile) workgroup of the plan: a whole row, so every key group's block of
    head-dim columns and every prompt split's share is in it;
  * one whole (request, kv head) pair is compared in full;
  * scaled workloads are redrawn unscaled (where the softmax is far from
    uniform);
  * the bench's own call, one captured step of the survivor selection and a
    fused append + decode per layer, runs on the full-size semantic-ID and
    long-history workloads: tables, lengths and pool rows bit-exact against
    the append oracle (with the selected parents), the selection bit-exact
    against its oracle, outputs against the attention oracle.
The tiny fp32 workload is checked in full.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from generative_recommendation_beam_amd import device as dv
from generative_recommendation_beam_amd import inputs, xattn
from oracle import append as oapp
from oracle import attention as oa
from oracle import beam_topk as obt
from parity import compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    xattn.lib()


def _np(t):
    return t.detach().cpu().numpy()


def workgroup_rows(w, plan, seed):
    """One (beam, query head) row inside every (request, kv head, row tile)
    of the plan, at a seeded position within the tile."""
    rng = np.random.default_rng(seed)
    G = w.Hq // w.Hkv
    M = w.B * G
    rpb = plan["rows_per_block"] or M
    tiles = plan["row_tiles"] or 1
    rows = []
    for r in range(w.R):
        for h in range(w.Hkv):
            for t in range(tiles):
                lo = t * rpb
                hi = min(M, lo + rpb)
                if lo >= hi:
                    continue
                i = int(rng.integers(lo, hi))
                rows.append((r * w.B + i // G, h * G + i % G))
    rows += [(0, 0), (w.N_b - 1, w.Hq - 1)]
    return rows


def pair_rows(w, r, h):
    G = w.Hq // w.Hkv
    return [(r * w.B + b, h * G + g) for b in range(w.B) for g in range(G)]


def check_rows(w, o, lse, rows, what):
    O, L = oa.attention_rows(w, rows)
    og = np.stack([o[n, q] for n, q in rows])
    lg = np.array([lse[n, q] for n, q in rows])
    return compare(og, O, lg, L, w.dtype, what)


def run_cfg(cfg, unscaled=False, full_pair=True):
    w = inputs.config(cfg, unscaled=unscaled)
    print(f"[cfg {cfg} unscaled={unscaled}] R={w.R} B={w.B} P={int(w.prefix_len.max())} "
          f"L={w.unshared_len.tolist()[:4]} Hq={w.Hq} Hkv={w.Hkv}", flush=True)
    d = dv.upload(w)
    dv.build_cache(d)
    o, lse, ws, nb = dv.alloc_outputs(d, 2)
    o.fill_(float("nan"))
    lse.fill_(float("nan"))
    dv.decode(d, o, lse, ws, nb)
    torch.cuda.synchronize()
    o = _np(o)[:d.rows].reshape(w.N_b, w.Hq, w.D)
    lse = _np(lse)[:d.rows].reshape(w.N_b, w.Hq)
    assert np.isfinite(o).all() and np.isfinite(lse).all(), f"config {cfg}: rows left unwritten or non-finite"
    plan = xattn.get_plan(d.dims, 2)
    rows = workgroup_rows(w, plan, seed=400)
    stats = check_rows(w, o, lse, rows, f"config {cfg} unscaled={unscaled}: one row per workgroup ({len(rows)})")
    if full_pair:
        r, h = w.R - 1, w.Hkv // 2
        check_rows(w, o, lse, pair_rows(w, r, h), f"config {cfg} unscaled={unscaled}: whole pair (r={r}, h={h})")
    return w, o, lse, stats


def test_config1_full():
    w = inputs.config(1)
    d = dv.upload(w)
    dv.build_cache(d)
    o, lse, ws, nb = dv.alloc_outputs(d, 2)
    o.fill_(float("nan"))
    lse.fill_(float("nan"))
    dv.decode(d, o, lse, ws, nb)
    torch.cuda.synchronize()
    O, L = oa.attention(w)
    compare(_np(o)[:d.rows].reshape(O.shape), O, _np(lse)[:d.rows].reshape(L.shape), L, "f32",
            "config 1")


@pytest.mark.parametrize("cfg", [2, 3, "4A", "4B", "4B2g", "4B2i", "4B2d", 5])
def test_config_every_workgroup(cfg):
    run_cfg(cfg)


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_config_unscaled_every_workgroup(cfg):
    run_cfg(cfg, unscaled=True)


def test_config4_homogeneous_equals_heterogeneous():
    _, oa_, la, _ = run_cfg("4A", full_pair=False)
    _, ob_, lb, _ = run_cfg("4B", full_pair=False)
    compare(oa_, ob_, la, lb, "bf16", "4A vs 4B")


@pytest.mark.parametrize("cfg", ["4B2i", "4B2d"])
def test_config4_homogeneous_equals_aliased(cfg):
    """Aliased prompt offsets (interleaved order; one private copy) read the
    same values as the homogeneous batch: outputs match it row for row,
    permuted to the aliased request order."""
    _, oa_, la, _ = run_cfg("4A", full_pair=False)
    w, ob_, lb, _ = run_cfg(cfg, full_pair=False)
    seq = np.array(w.meta["seq_of_request"])
    compare(ob_, oa_[seq], lb, la[seq], "bf16", f"4A vs {cfg}")


# ------------------------------------------------ the bench's step at full size

def _oracle_cache(w, steps):
    """Append oracle over the first `steps` decode steps (in place)."""
    kpool = np.zeros((max(w.num_slots, 1), w.Hkv, w.D), dtype=w.k_new.dtype)
    vpool = np.zeros_like(kpool)
    table = np.full((w.N_b, w.T_max), -1, dtype=np.int64)
    ulen = np.zeros(w.R, dtype=np.int64)
    for t in range(steps):
        oapp.cache_append(B=w.B, k_new=w.k_new[t], v_new=w.v_new[t], parent=w.parents[t],
                          slot_base=w.slot_base, active=w.active(t), k_pool=kpool, v_pool=vpool,
                          table_in=table, table_out=table, unshared_len=ulen)
    return kpool, vpool, table, ulen


@pytest.mark.parametrize("cfg", [2, 5])
def test_bench_step_graph_full_size(cfg):
    """The call bench.py times, at full size: the survivor selection over the
    beam_width x top_k pool, then one fused xattn_append_decode per layer
    (ping-pong tables) reading the selected parents, captured as one graph
    and replayed twice (lengths restored, outputs poisoned in between)."""
    w = inputs.config(cfg)
    print(f"[bench step cfg {cfg}] R={w.R} B={w.B} P={int(w.prefix_len.max())} L={w.T_steps}", flush=True)
    d = dv.upload(w)
    table_in, table_out, t_last = dv.prepare_step(d)
    assert t_last is not None
    o, lse, ws, nb = dv.alloc_outputs(d, 3)
    plan = xattn.get_plan(d.dims, 2)
    assert plan["mfma"] == 1 and plan["partials"] == 0 and plan["launches"] == 1, plan  # the folded append
    K = max(1, min(w.B, 512))
    x = inputs.make_topk("select", R=w.R, BW=w.B, K=K, n_out=w.B, seed_key=(700, 0))
    P_sel, T_sel, S_sel = obt.select(x.beam_score, x.logprob, x.token, x.n_out)
    sel_in = [torch.from_numpy(v).cuda() for v in (x.beam_score, x.logprob, x.token)]
    parent = torch.empty((w.R, w.B), dtype=torch.int32, device="cuda")
    tok = torch.empty_like(parent)
    sc = torch.empty((w.R, w.B), dtype=torch.float32, device="cuda")
    st = dv.layer_step(d, o, lse, ws, nb, table_in, table_out, t_last)
    st.parent = parent.data_ptr()
    g = xattn.StepGraph([st], select=xattn.beam_select(*sel_in, w.B, parent, tok, sc))
    # oracle state: every step but the last with the workload's parents, the
    # last with the selected ones
    w.parents[t_last] = P_sel.reshape(-1)
    kp, vp, tab, ul = _oracle_cache(w, w.T_steps)
    u0 = d.unshared_len.clone()
    try:
        for rep in range(2):
            d.unshared_len.copy_(u0)
            parent.fill_(-1)
            o.fill_(float("nan"))
            lse.fill_(float("nan"))
            torch.cuda.synchronize()
            g.launch()
            torch.cuda.synchronize()
            assert np.array_equal(_np(parent), P_sel) and np.array_equal(_np(tok), T_sel)
            assert np.array_equal(_np(sc).view(np.uint32), S_sel.view(np.uint32))
            assert np.array_equal(_np(d.unshared_len)[:w.R], ul), f"replay {rep}: lengths"
            assert np.array_equal(_np(table_out).astype(np.int64), tab), f"replay {rep}: slot table"
            assert np.array_equal(_np(d.k_pool.view(torch.int16)), kp.view(np.int16)), f"replay {rep}: K pool"
            assert np.array_equal(_np(d.v_pool.view(torch.int16)), vp.view(np.int16)), f"replay {rep}: V pool"
            og = _np(o)[:d.rows].reshape(w.N_b, w.Hq, w.D)
            lg = _np(lse)[:d.rows].reshape(w.N_b, w.Hq)
            assert np.isfinite(og).all() and np.isfinite(lg).all(), f"replay {rep}: rows left unwritten"
            check_rows(w, og, lg, workgroup_rows(w, plan, seed=410 + rep),
                       f"bench step cfg {cfg} replay {rep}: one row per workgroup")
        r, h = 0, w.Hkv - 1
        check_rows(w, og, lg, pair_rows(w, r, h), f"bench step cfg {cfg}: whole pair (r={r}, h={h})")
    finally:
        g.close()
