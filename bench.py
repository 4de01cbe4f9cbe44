"""Benchmark: staged beam-search decode attention on one MI355X.

One step = one decode step: xattn_beam_topk picks each request's surviving
beams from its beam_width x top_k candidate pool, then per layer the cache
append of the step's new tokens (token-granular K/V write and slot-table
rewrite, with the selected parents) and the decode, as one
xattn_append_decode call (ping-pong tables; the append folds into the decode
launch), on n_layers distinct layer buffers (distinct Q, prompt KV,
Non-Shared pool, slot tables and lengths per layer, so the working set
defeats the 256 MB Infinity Cache). By default the whole step is one
captured HIP graph (xattn_step_graph_*), launched once per step; --eager
launches every call from the host instead. Inputs are synthetic, shaped like
the GR semantic-ID workload by default (8 requests, 1024-token user-history
prompt, beam width 128, 3 generated tokens, 16 q / 4 kv heads, head dim 128,
bf16), and resident in HBM before the timed region; the cache holds every
earlier step, and each timed step restores the lengths (one small device
copy) and appends the last step's tokens again, so every step does the same
work.

Prints ONE JSON line. Metric: beams * layer-steps per second, plus achieved
HBM bandwidth on algorithmic bytes (unique KV: prompt KV once per request,
generated KV once per beam; plus the append's new rows and table cells) and
the roofline of the dominant kernel (the fused append + decode launch). Its
per-launch duration comes from HIP events: around every call of the timed
steps with --eager; in graph mode, around K launches of a graph of every
layer's call, right after the timed steps, each after the lengths are
restored (events cannot be recorded inside a captured graph on the runtime
PyTorch ships).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # fp32 vector

DEFAULT_LAYERS = {"1": 16, "2": 16, "3": 6, "4A": 3, "4B": 2, "4B2g": 2, "4B2i": 2, "4B2d": 2, "5": 2}
WORKLOAD_NAMES = {
    "1": "tiny fp32: R=1 P=256 B=4 L=2 4q/1kv D=64",
    "2": "GR semantic-ID decode: R=8 P=1024 B=128 L=3 16q/4kv D=128 bf16",
    "3": "wide beam: R=4 P=2048 B=512 L=1-3 32q/8kv D=128 bf16",
    "4A": "prefix-homogeneous: 4 prefixes x 16 seqs P=4096 +512 unique, 32q/8kv D=128 bf16",
    "4B": "prefix-heterogeneous: 64 prefixes P=4096 +512 unique, 32q/8kv D=128 bf16",
    "4B2g": "64 single-sequence requests on 4 aliased prefixes, grouped order, P=4096 +512 unique, 32q/8kv D=128 bf16",
    "4B2i": "64 single-sequence requests on 4 aliased prefixes, interleaved order, P=4096 +512 unique, 32q/8kv D=128 bf16",
    "4B2d": "as 4B2g with one request on a private prefix copy (one divergent request), 32q/8kv D=128 bf16",
    "5": "long history: R=16 P=16384 B=256 L=8 64q/8kv D=128 bf16",
}


def _cfg_key(s):
    return int(s) if s.isdigit() else s


def algorithmic(w):
    """Algorithmic bytes / flops of one decode call on workload w."""
    e = w.elem_bytes
    # prompt rows once per distinct physical range (requests may alias one prefix)
    prompt_tokens = sum(p for (o, p) in {(int(w.prefix_off[r]), int(w.prefix_len[r])) for r in range(w.R)})
    kv_tokens = prompt_tokens + int(sum(w.B * int(w.unshared_len[r]) for r in range(w.R)))
    unique_kv = kv_tokens * w.Hkv * w.D * 2 * e
    q = w.N_b * w.Hq * w.D * e
    out = w.N_b * w.Hq * (w.D + 1) * 4
    slots = int(sum(w.B * int(w.unshared_len[r]) for r in range(w.R))) * 4
    total = unique_kv + q + out + slots
    mfma_flops = 4 * w.D * w.Hq * int(sum(w.B * int(w.prefix_len[r]) for r in range(w.R)))
    all_flops = 4 * w.D * w.Hq * int(sum(w.B * (int(w.prefix_len[r]) + int(w.unshared_len[r])) for r in range(w.R)))
    return dict(unique_kv=unique_kv, total=total, mfma_flops=mfma_flops, flops=all_flops)


def _oracle_state(w):
    """Oracle cache state before the last step's append (untimed set-up)."""
    import numpy as np
    from oracle import append as oapp
    kpool = np.zeros((max(w.num_slots, 1), w.Hkv, w.D), dtype=w.k_new.dtype)
    vpool = np.zeros_like(kpool)
    table = np.full((w.N_b, w.T_max), -1, dtype=np.int64)
    ulen = np.zeros(w.R, dtype=np.int64)
    for t in range(max(w.T_steps - 1, 0)):
        oapp.cache_append(B=w.B, k_new=w.k_new[t], v_new=w.v_new[t], parent=w.parents[t],
                          slot_base=w.slot_base, active=w.active(t), k_pool=kpool, v_pool=vpool,
                          table_in=table, table_out=table, unshared_len=ulen)
    return kpool, vpool, table, ulen


def cpu_baseline(layers_np, min_seconds=10.0):
    """Time the oracle (as it stands) on whole layer steps, the append of the
    last step's tokens plus the decode attention, until min_seconds pass."""
    from oracle import append as oapp
    from oracle import pool
    states = [_oracle_state(w) for w in layers_np]
    done_beams = 0
    done_layers = 0
    workers = pool.host_cores()
    used = workers
    t0 = time.perf_counter()
    i = 0
    while True:
        w = layers_np[i % len(layers_np)]
        kpool, vpool, table, ulen = states[i % len(layers_np)]
        if w.T_steps > 0:
            t = w.T_steps - 1
            u0 = ulen.copy()
            tout = table.copy()
            oapp.cache_append(B=w.B, k_new=w.k_new[t], v_new=w.v_new[t], parent=w.parents[t],
                              slot_base=w.slot_base, active=w.active(t), k_pool=kpool, v_pool=vpool,
                              table_in=table, table_out=tout, unshared_len=ulen)
            ulen[:] = u0
        _, _, dt, used = pool.attention_parallel(w, workers=workers)
        done_beams += w.N_b
        done_layers += 1
        i += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    el = time.perf_counter() - t0
    return dict(value=done_beams / el, unit="beams*layer-steps/s", cores=used, kind="oracle",
                sample=f"{done_layers} full layer steps (append of the last step's tokens + decode) "
                       f"of the same workload (fp64 numpy oracle, {used} worker processes, {el:.1f} s)")


def paged_baseline(layers, K, xattn_decode_us, xattn_call_us, xattn_step_ms):
    """The same layers in a PagedAttention-style block-paged cache: per layer,
    the copies branching beams make of their partial tail blocks, then the
    per-beam paged decode. HIP events around every call, K rounds, queued
    behind each other (each call outlasts its host launch)."""
    import numpy as np
    import torch
    from generative_recommendation_beam_amd import device as dv
    from generative_recommendation_beam_amd import xattn
    paged = []
    for (d, o, lse, ws, nb, tin, tout, t_last) in layers:
        pc = dv.build_paged(d, tout)
        pnb = xattn.paged_workspace_size(d.dims, pc.max_seq_len)
        pws = torch.zeros(max(pnb, 1), dtype=torch.uint8, device="cuda")
        paged.append((d, pc, o, lse, pws, pnb))
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    rounds = [[(ev(), ev(), ev()) for _ in paged] for _ in range(K)]
    for d, pc, o, lse, pws, pnb in paged:  # warm-up
        xattn.paged_copy_blocks(d.dims, pc.k_cache, pc.v_cache, pc.parent_tail, pc.spare)
        dv.paged_decode(d, pc, o, lse, pws, pnb)
    torch.cuda.synchronize()
    start, end = ev(), ev()
    start.record()
    for r in rounds:
        for (d, pc, o, lse, pws, pnb), (e0, e1, e2) in zip(paged, r):
            e0.record()
            xattn.paged_copy_blocks(d.dims, pc.k_cache, pc.v_cache, pc.parent_tail, pc.spare)
            e1.record()
            dv.paged_decode(d, pc, o, lse, pws, pnb)
            e2.record()
    end.record()
    torch.cuda.synchronize()
    copy_us = float(np.mean([[e0.elapsed_time(e1) for e0, e1, e2 in r] for r in rounds]) * 1e3)
    dec_us = float(np.mean([[e1.elapsed_time(e2) for e0, e1, e2 in r] for r in rounds]) * 1e3)
    step_ms = start.elapsed_time(end) / K
    pc0 = paged[0][1]
    return dict(decode_us_per_call=round(dec_us, 2), block_copy_us_per_call=round(copy_us, 2),
                step_ms=round(step_ms, 4), blocks_per_layer=int(pc0.k_cache.shape[0]),
                decode_speedup_xattn=round(dec_us / xattn_decode_us, 2),
                layer_speedup_xattn=round((copy_us + dec_us) / xattn_call_us, 2),
                step_speedup_xattn=round(step_ms / xattn_step_ms, 2),
                note="same layers, same attention; PagedAttention-style per-beam paged decode "
                     "(16-token blocks, prompt blocks shared and re-read by every beam) plus the "
                     "copy each beam makes of its parent's tail block; eager launches. "
                     "decode_speedup_xattn: against xattn's decode alone; layer_speedup_xattn: "
                     "copy + decode against the fused append + decode call")


def batch_former_timing():
    """Host batch former (xattn_cht_*) on the Feather page's sensitivity
    shape: 800 requests in 8 shuffled prefix groups, 1024-token prefixes plus
    128 unique tokens, 16-token blocks; batches of up to 100 formed and
    retired until none wait."""
    import random
    from generative_recommendation_beam_amd import xattn
    rng = random.Random(11)
    bs = 16
    groups = [[rng.randint(0, 30000) for _ in range(1024)] for _ in range(8)]
    order = [g for g in range(8) for _ in range(100)]
    rng.shuffle(order)
    reqs = [groups[g] + [rng.randint(0, 30000) for _ in range(128)] for g in order]
    c = xattn.Cht(bs)
    t0 = time.perf_counter()
    for rid, toks in enumerate(reqs):
        c.insert(rid, toks)
    t1 = time.perf_counter()
    batches, homogeneous = 0, 0
    t_form = 0.0
    while True:
        s0 = time.perf_counter()
        b = c.form_batch(100, 128 // bs)
        t_form += time.perf_counter() - s0
        if not b:
            break
        batches += 1
        homogeneous += len({order[r] for r in b}) == 1
        s0 = time.perf_counter()
        for r in b:
            c.complete(r)
        t_form += time.perf_counter() - s0
    c.close()
    return dict(requests=len(reqs), insert_us_per_request=round((t1 - t0) / len(reqs) * 1e6, 2),
                form_and_retire_us_per_request=round(t_form / len(reqs) * 1e6, 2), batches=batches,
                homogeneous_batches=homogeneous,
                note="host C++ through ctypes (the per-call Python overhead included)")


def append_bytes(w):
    """Algorithmic bytes of one layer's append of the last step's tokens."""
    e = w.elem_bytes
    if w.T_steps == 0:
        return 0
    t = w.T_steps - 1
    act = w.active(t)
    beams = int(sum(w.B for r in range(w.R) if act[r]))
    return 2 * 2 * beams * w.Hkv * w.D * e + 2 * beams * t * 4 + beams * 4


KERNEL_SOURCES = ("generative_recommendation_beam_amd/csrc/shared_mfma.hip",
                  "generative_recommendation_beam_amd/csrc/device.h",
                  "generative_recommendation_beam_amd/csrc/kernels.h",
                  "generative_recommendation_beam_amd/csrc/api.cpp")


def kernel_hash():
    """Hash of the sources of the Shared-stage kernel and its launch plan."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(cfg):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    counts, each scaled by the same counter's reading for a plain copy of known
    size; None if absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    e = t.get("workloads", {}).get(str(cfg))
    if not e or e.get("kernel_hash") != kernel_hash():
        return None
    cal = t["copy_calibration"]
    return int(e["fetch_kib"] * 1024 * cal["fetch_factor"] + e["write_kib"] * 1024 * cal["write_factor"])


def calibrate_copy(nbytes, reps):
    """A plain device copy of known size, for scaling byte counters."""
    import torch
    torch.cuda.set_device(0)
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="2")
    ap.add_argument("--layers", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--prefix-splits", type=int, default=0, help="override the split plan (0 = auto)")
    ap.add_argument("--rows-per-block", type=int, default=0, help="override rows per workgroup (0 = auto)")
    ap.add_argument("--stages", type=int, default=0, help="override LDS pipeline stages (0 = auto)")
    ap.add_argument("--key-groups", type=int, default=0, help="override key groups per workgroup (0 = auto)")
    ap.add_argument("--no-paged", action="store_true",
                    help="skip the PagedAttention-style baseline measured beside the step")
    ap.add_argument("--eager", action="store_true",
                    help="launch every call from the host instead of one captured step graph")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, 3)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(requests shard across GPUs with no exchange; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from generative_recommendation_beam_amd import device as dv
    from generative_recommendation_beam_amd import inputs, xattn

    if not os.path.exists(xattn.LIB_PATH):
        from generative_recommendation_beam_amd import build as _b
        _b.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    cfg = _cfg_key(args.config)
    n_layers = args.layers or DEFAULT_LAYERS[str(cfg)]

    layers_np = [inputs.config(cfg, layer=l) for l in range(n_layers)]
    w0 = layers_np[0]
    # One [n_layers][R] length array, restored with one copy per step.
    ulen_all = torch.zeros((n_layers, max(w0.R, 1)), dtype=torch.int32, device="cuda")
    layers = []
    for l, w in enumerate(layers_np):
        d = dv.upload(w, prefix_splits=args.prefix_splits, rows_per_block=args.rows_per_block,
                      pipeline_stages=args.stages, key_groups=args.key_groups)
        d.unshared_len = ulen_all[l]
        table_in, table_out, t_last = dv.prepare_step(d)
        o, lse, ws, nb = dv.alloc_outputs(d, 3 if t_last is not None else 2)
        layers.append((d, o, lse, ws, nb, table_in, table_out, t_last))
    ulen0 = ulen_all.clone()
    # The step opens with the survivor selection (beam width x top-k pool per
    # request, top-k = beam width) whose parents every layer's append reads.
    topk_k = max(1, min(w0.B, 512))
    tx = inputs.make_topk("select", R=w0.R, BW=w0.B, K=topk_k, n_out=w0.B, seed_key=(700, 0))
    sel_in = [torch.from_numpy(v).cuda() for v in (tx.beam_score, tx.logprob, tx.token)]
    sel_parent = torch.empty((w0.R, w0.B), dtype=torch.int32, device="cuda")
    sel_tok = torch.empty_like(sel_parent)
    sel_score = torch.empty((w0.R, w0.B), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    plan = xattn.get_plan(layers[0][0].dims, 2)
    alg = algorithmic(w0)
    K = args.steps

    def new_events():
        return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in layers]

    def eager_step(evs):
        ulen_all.copy_(ulen0)
        xattn.beam_topk(*sel_in, w0.B, sel_parent, sel_tok, sel_score)
        for (d, o, lse, ws, nb, tin, tout, t_last), (e0, e1) in zip(layers, evs):
            e0.record()
            if t_last is not None:
                xattn.append_decode(d.dims, q=d.q, k_shared=d.k_shared, v_shared=d.v_shared,
                                    prefix_off=d.prefix_off, prefix_len=d.prefix_len, k_new=d.k_new[t_last],
                                    v_new=d.v_new[t_last], parent=sel_parent, slot_base=d.slot_base,
                                    active=d.active[t_last], k_pool=d.k_pool, v_pool=d.v_pool, table_in=tin,
                                    table_out=tout, unshared_len=d.unshared_len, o=o, lse=lse,
                                    workspace=ws if nb else None, workspace_bytes=nb)
            else:
                xattn.decode(d.dims, d.q, d.k_shared, d.v_shared, d.prefix_off, d.prefix_len, d.k_pool,
                             d.v_pool, tout, d.unshared_len, o, lse, ws if nb else None, nb)
            e1.record()

    step_evs = [new_events() for _ in range(K)] if args.eager else []
    warm_evs = new_events()
    if not args.eager:
        # The whole step (every layer's append and decode) as one graph.
        steps = []
        for (d, o, lse, ws, nb, tin, tout, t_last) in layers:
            st = dv.layer_step(d, o, lse, ws, nb, tin, tout, t_last)
            st.parent = sel_parent.data_ptr()
            steps.append(st)
        select = xattn.beam_select(*sel_in, w0.B, sel_parent, sel_tok, sel_score)
        step_graph = xattn.StepGraph(steps, select=select)
        select_graph = xattn.StepGraph([], select=xattn.beam_select(*sel_in, w0.B, sel_parent, sel_tok,
                                                                    sel_score))
        # Every layer's call alone, back to back in one graph, to time the
        # dominant kernel with HIP events around its launches (the runtime
        # PyTorch ships cannot record events inside a captured graph); and
        # the plain decodes on the complete caches, for reference.
        layer_graph = xattn.StepGraph(steps)
        decode_graph = xattn.StepGraph([dv.layer_step(d, o, lse, ws, nb, None, tout, None)
                                        for (d, o, lse, ws, nb, tin, tout, t_last) in layers])
        torch.cuda.synchronize()

    def one_step(k):
        if args.eager:
            eager_step(warm_evs if k < 0 else step_evs[k])
        else:
            ulen_all.copy_(ulen0)
            step_graph.launch()

    for _ in range(args.warmup):
        one_step(-1)
    torch.cuda.synchronize()

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for k in range(K):
        one_step(k)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(end)
    select_us = None
    decode_only_us = None
    if args.eager:
        call_ms = np.array([[e0.elapsed_time(e1) for (e0, e1) in evs] for evs in step_evs])
        call_us = float(call_ms.mean() * 1e3)
    else:
        # Kernel timing pass, right after the timed steps, on the state they
        # leave (every layer's cache complete): K launches of the graph of
        # every layer's decode, each between two HIP events on the launch
        # stream; a decode's duration is the pair's interval / n_layers
        # (back-to-back kernels of one graph: only graph-internal gaps added).
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(K)]
        for e0, e1 in pairs:
            ulen_all.copy_(ulen0)  # the same append every launch
            e0.record()
            layer_graph.launch()
            e1.record()
        dpairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(K)]
        for e0, e1 in dpairs:
            e0.record()
            decode_graph.launch()
            e1.record()
        spairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(K)]
        for e0, e1 in spairs:
            e0.record()
            select_graph.launch()
            e1.record()
        torch.cuda.synchronize()
        call_us = float(np.mean([e0.elapsed_time(e1) for e0, e1 in pairs]) * 1e3 / n_layers)
        decode_only_us = float(np.mean([e0.elapsed_time(e1) for e0, e1 in dpairs]) * 1e3 / n_layers)
        select_us = float(np.mean([e0.elapsed_time(e1) for e0, e1 in spairs]) * 1e3)
        step_graph.close()
        layer_graph.close()
        decode_graph.close()
        select_graph.close()

    ms_per_step = ms_total / K
    value = w0.N_b * n_layers / (ms_per_step / 1e3)
    # The timed call is the fused append + decode when the layers append
    # (one launch when the plan folds the append in): its bytes include the
    # append's.
    appends = layers[0][7] is not None
    fused = appends and plan["mfma"] == 1 and plan["partials"] == 0
    call_bytes = alg["total"] + (append_bytes(w0) if appends else 0)
    t_hbm = call_bytes / (PEAK_HBM_GBS * 1e9)
    peak_tflops = PEAK_BF16_TFLOPS if w0.dtype == "bf16" else PEAK_FP32_TFLOPS
    t_mfma = alg["mfma_flops"] / (peak_tflops * 1e12)
    call_s = call_us * 1e-6
    if t_hbm >= t_mfma:
        achieved = call_bytes / call_s / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(achieved / PEAK_HBM_GBS, 4), traffic=measured_traffic(cfg))
    else:
        achieved = alg["mfma_flops"] / call_s / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=peak_tflops, unit="TFLOP/s",
                    frac=round(achieved / peak_tflops, 4), traffic=measured_traffic(cfg))
    if fused:
        roof["kernel"] = "xattn_append_decode call (1 kernel launch: the append folded into the decode)"
    elif appends:
        roof["kernel"] = "xattn_append_decode call (append, then %d decode launch%s)" % (
            plan["launches"], "" if plan["launches"] == 1 else "es")
    else:
        roof["kernel"] = "xattn_decode call (%d kernel launch%s)" % (plan["launches"], "" if plan["launches"] == 1 else "es")
    roof["timing"] = ("HIP events around K launches of a graph of the n_layers calls (interval / "
                      "n_layers; lengths restored before each launch, outside the events), run right "
                      "after the timed steps" if not args.eager else
                      "HIP events around every call of the timed steps")
    roof["avg_call_us"] = round(call_us, 3)
    if decode_only_us is not None:
        roof["decode_only_us"] = round(decode_only_us, 3)
    roof["algorithmic_bytes_per_call"] = call_bytes
    roof["algorithmic_mfma_flops_per_call"] = alg["mfma_flops"]
    roof["kernel_hash"] = kernel_hash()

    result = {
        "metric": "beam-decode attention beams*layer-steps/s; achieved HBM GB/s vs peak",
        "value": round(value, 1),
        "unit": "beams*layer-steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w0.dtype,
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[str(cfg)], "n_layers": n_layers,
                   "beams_per_call": w0.N_b,
                   "step": "beam selection (%d x %d x %d pool -> %d beams per request), then "
                           "append + decode per layer (one xattn_append_decode call)" % (w0.R, w0.B, topk_k, w0.B),
                   "launch": "eager" if args.eager else "graph", "plan": plan},
        "unique_kv_GBps": round(alg["unique_kv"] / call_s / 1e9, 1),
        "total_GBps": round(call_bytes / call_s / 1e9, 1),
        "mfma_TFLOPs": round(alg["mfma_flops"] / call_s / 1e12, 1),
        "wall_s_timed": round(wall, 4),
        "step_GBps": round(n_layers * (alg["total"] + append_bytes(w0)) / (ms_per_step * 1e-3) / 1e9, 1),
        "roofline": roof,
        "beam_select_us": None if select_us is None else round(select_us, 3),
    }
    if not args.no_paged and w0.dtype == "bf16":
        print("timing the PagedAttention-style baseline ...", file=sys.stderr, flush=True)
        result["paged_baseline"] = paged_baseline(layers, K, decode_only_us or call_us, call_us, ms_per_step)
    result["batch_former"] = batch_former_timing()
    if not args.no_cpu_baseline:
        print("timing the oracle on host cores ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(layers_np, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
