"""Graph-captured multi-layer decode step (append + decode per layer) through
the C-ABI, checked against the fp64 oracle on every replay (needs an MI355X).

Each layer holds a different workload (different dims), so the graph carries
per-layer parameters. Between replays the lengths are restored and the
outputs poisoned with eager work, and every replay is checked.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from generative_recommendation_beam_amd import device as dv
from generative_recommendation_beam_amd import xattn
from generative_recommendation_beam_amd.inputs import make_topk, make_workload
from oracle import append as oapp
from oracle import attention as oa
from oracle import beam_topk as bt
from parity import compare

pytestmark = pytest.mark.gpu

LAYERS = [
    dict(R=2, B=16, Hq=8, Hkv=2, D=128, prefix_len=[500, 200], unshared_len=[3, 2]),
    dict(R=3, B=8, Hq=4, Hkv=1, D=64, prefix_len=[130, 0, 64], unshared_len=[2, 1, 3]),
    dict(R=2, B=40, Hq=16, Hkv=4, D=128, prefix_len=[700, 1100], unshared_len=[1, 4]),
    dict(R=1, B=4, Hq=4, Hkv=1, D=64, prefix_len=[256], unshared_len=[2], dtype="f32"),
    # long generated tails: the prompt pass (with the append), then a
    # Non-Shared pass of its own that folds the prompt's partials in
    dict(R=2, B=4, Hq=8, Hkv=2, D=128, prefix_len=[600, 300], unshared_len=[40, 20]),
    dict(R=2, B=3, Hq=4, Hkv=1, D=64, prefix_len=[0, 150], unshared_len=[30, 25]),
]
LONG_TAIL = [4, 5]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    xattn.lib()


def _np(t):
    return t.detach().cpu().numpy()


def _oracle_cache(w):
    kpool = np.zeros((w.num_slots, w.Hkv, w.D), dtype=w.k_new.dtype)
    vpool = np.zeros_like(kpool)
    table = np.full((w.N_b, w.T_max), -1, dtype=np.int64)
    ulen = np.zeros(w.R, dtype=np.int64)
    for t in range(w.T_steps):
        oapp.cache_append(B=w.B, k_new=w.k_new[t], v_new=w.v_new[t], parent=w.parents[t],
                          slot_base=w.slot_base, active=w.active(t), k_pool=kpool, v_pool=vpool,
                          table_in=table, table_out=table, unshared_len=ulen)
    return kpool, vpool, table, ulen


def _bits(t):
    return _np(t.view(torch.int16)) if t.dtype == torch.bfloat16 else _np(t)


def test_step_graph_every_replay_matches_oracle():
    ws_, ds, outs, steps, ulen0, refs = [], [], [], [], [], []
    for i, kw in enumerate(LAYERS):
        w = make_workload(f"step{i}", seed_key=(320, i), **kw)
        d = dv.upload(w)
        table_in, table_out, t_last = dv.prepare_step(d)
        o, lse, ws, nb = dv.alloc_outputs(d, 3)
        steps.append(dv.layer_step(d, o, lse, ws, nb, table_in, table_out, t_last))
        ws_.append(w)
        ds.append((d, table_out))
        outs.append((o, lse, ws))   # every buffer the graph refers to stays alive
        ulen0.append(d.unshared_len.clone())
        refs.append((oa.attention(w), _oracle_cache(w)))
    g = xattn.StepGraph(steps)
    try:
        for rep in range(3):
            for (d, _), (o, lse, _ws), u0 in zip(ds, outs, ulen0):
                d.unshared_len.copy_(u0)
                o.fill_(float("nan"))
                lse.fill_(float("nan"))
            torch.cuda.synchronize()
            g.launch()
            torch.cuda.synchronize()
            for w, (d, table_out), (o, lse, _ws), ((O, L), (kp, vp, tab, ul)) in zip(ws_, ds, outs, refs):
                compare(_np(o)[:d.rows].reshape(O.shape), O, _np(lse)[:d.rows].reshape(L.shape), L,
                        w.dtype, f"step graph replay {rep} {w.name}")
                assert np.array_equal(_np(d.unshared_len)[:w.R], ul)
                assert np.array_equal(_np(table_out).astype(np.int64), tab)
                assert np.array_equal(_bits(d.k_pool), kp.view(np.int16) if w.dtype == "bf16" else kp)
                assert np.array_equal(_bits(d.v_pool), vp.view(np.int16) if w.dtype == "bf16" else vp)
    finally:
        g.close()


@pytest.mark.parametrize("li", [0] + LONG_TAIL)
def test_step_graph_equals_eager_bitwise(li):
    """A replay gives the same bits as the eager calls it captured (for the
    long tails: the prompt pass with the append, then the Non-Shared pass
    that merges everything)."""
    kw = LAYERS[li]
    w = make_workload("stepE", seed_key=(321, li), **kw)
    d = dv.upload(w)
    table_in, table_out, t_last = dv.prepare_step(d)
    u0 = d.unshared_len.clone()
    o, lse, ws, nb = dv.alloc_outputs(d, 3)
    plan = xattn.get_plan(d.dims, 2)
    if li in LONG_TAIL:
        assert plan["unshared_splits"] > 0 and plan["partials"] > 0, plan
    g = xattn.StepGraph([dv.layer_step(d, o, lse, ws, nb, table_in, table_out, t_last)])
    try:
        g.launch()
        torch.cuda.synchronize()
        og, lg = _np(o).copy(), _np(lse).copy()
        d.unshared_len.copy_(u0)
        dv.append_step(d, t_last, table_in=table_in, table_out=table_out)
        xattn.decode(d.dims, d.q, d.k_shared, d.v_shared, d.prefix_off, d.prefix_len, d.k_pool,
                     d.v_pool, table_out, d.unshared_len, o, lse, ws if nb else None, nb)
        torch.cuda.synchronize()
        assert np.array_equal(og, _np(o)) and np.array_equal(lg, _np(lse))
    finally:
        g.close()


def test_step_graph_rejects_bad_layer_without_keeping_anything():
    w = make_workload("stepBad", seed_key=(322, 0), **LAYERS[0])
    d = dv.upload(w)
    table_in, table_out, t_last = dv.prepare_step(d)
    o, lse, ws, nb = dv.alloc_outputs(d, 3)
    good = dv.layer_step(d, o, lse, ws, nb, table_in, table_out, t_last)
    bad = dv.layer_step(d, o, lse, ws, nb, table_in, table_out, t_last)
    bad.q = None
    with pytest.raises(xattn.XattnError) as e:
        xattn.StepGraph([good, bad])
    assert e.value.status == xattn.XATTN_ERR_INVALID_ARG
    # the stream is usable afterwards
    g = xattn.StepGraph([good])
    g.launch()
    torch.cuda.synchronize()
    g.close()


def test_decode_only_graph_timed_with_events():
    """A layer step with no append captures the decode alone; HIP events
    recorded around its launches time it (how the benchmark times the
    decode kernel)."""
    w = make_workload("stepT", seed_key=(323, 0), **LAYERS[2])
    d = dv.upload(w)
    dv.build_cache(d)
    o, lse, ws, nb = dv.alloc_outputs(d, 2)
    g = xattn.StepGraph([dv.layer_step(d, o, lse, ws, nb, None, d.table, None)])
    try:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.launch()
        e1.record()
        torch.cuda.synchronize()
        assert e0.elapsed_time(e1) > 0.0
        O, L = oa.attention(w)
        compare(_np(o)[:d.rows].reshape(O.shape), O, _np(lse)[:d.rows].reshape(L.shape), L, w.dtype,
                "decode-only graph")
    finally:
        g.close()


def test_step_graph_with_selection_feeds_every_layer():
    """Selection, then per layer append (with the selected parents) + decode,
    in one graph; checked on two replays against the oracle run on the same
    workloads with their last step's parents replaced by the oracle's
    selection."""
    R, B = 3, 24
    layers = [dict(R=R, B=B, Hq=8, Hkv=2, D=128, prefix_len=[300, 90, 700], unshared_len=[3, 3, 2]),
              dict(R=R, B=B, Hq=4, Hkv=1, D=64, prefix_len=[64, 200, 1], unshared_len=[3, 3, 2])]
    x = make_topk("sel", R=R, BW=B, K=20, n_out=B, seed_key=(324, 0))
    P, T, S = bt.select(x.beam_score, x.logprob, x.token, x.n_out)
    dev = "cuda"
    bs, lp, tk = (torch.from_numpy(a).to(dev) for a in (x.beam_score, x.logprob, x.token))
    parent = torch.empty((R, B), dtype=torch.int32, device=dev)
    tok = torch.empty((R, B), dtype=torch.int32, device=dev)
    sc = torch.empty((R, B), dtype=torch.float32, device=dev)
    sel = xattn.beam_select(bs, lp, tk, B, parent, tok, sc)
    state, steps = [], []
    for i, kw in enumerate(layers):
        w = make_workload(f"sel{i}", seed_key=(325, i), **kw)
        d = dv.upload(w)
        table_in, table_out, t_last = dv.prepare_step(d)
        o, lse, ws, nb = dv.alloc_outputs(d, 3)
        st = dv.layer_step(d, o, lse, ws, nb, table_in, table_out, t_last)
        st.parent = parent.data_ptr()   # the appends read the selection's output
        steps.append(st)
        w2 = make_workload(f"sel{i}", seed_key=(325, i), **kw)
        w2.parents[t_last] = P.reshape(-1)
        state.append((w2, d, table_out, o, lse, d.unshared_len.clone(), oa.attention(w2), _oracle_cache(w2)))
    g = xattn.StepGraph(steps, select=sel)
    try:
        for rep in range(2):
            parent.fill_(-1)
            for w2, d, table_out, o, lse, u0, _, _ in state:
                d.unshared_len.copy_(u0)
                o.fill_(float("nan"))
            torch.cuda.synchronize()
            g.launch()
            torch.cuda.synchronize()
            assert np.array_equal(_np(parent), P) and np.array_equal(_np(tok), T)
            assert np.array_equal(_np(sc).view(np.uint32), S.view(np.uint32))
            for w2, d, table_out, o, lse, u0, (O, L), (kp, vp, tab, ul) in state:
                compare(_np(o)[:d.rows].reshape(O.shape), O, _np(lse)[:d.rows].reshape(L.shape), L,
                        w2.dtype, f"selected step replay {rep} {w2.name}")
                assert np.array_equal(_np(table_out).astype(np.int64), tab)
                assert np.array_equal(_np(d.unshared_len)[:w2.R], ul)
    finally:
        g.close()
