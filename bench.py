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
launches every call from the host instead.

The default workload is the long-history one (16 requests, 16384-token
user-history prompt, beam width 256, 8 generated tokens, 64 q / 8 kv heads,
head dim 128, bf16: about 1 GB of prompt KV per layer), the largest
configuration that fits one GPU; the GR semantic-ID workload (8 requests,
1024-token prompt, beam width 128, 3 tokens, 16 q / 4 kv heads) is measured
in the same run as an extra block. Inputs are synthetic, resident in HBM
before the timed region; the cache holds every earlier step, and each timed
step restores the lengths (one small device copy) and appends the last
step's tokens again, so every step does the same work.

Prints ONE JSON line. Metric: beams * layer-steps per second, plus achieved
HBM bandwidth on algorithmic bytes (unique KV: prompt KV once per request,
generated KV once per beam; plus the append's new rows and table cells) and
the roofline of the dominant kernel (the fused append + decode launch). Its
per-launch duration comes from HIP events on the launch stream: around every
call of the timed steps with --eager; in graph mode, around K launches of a
graph of every layer's call, right after the timed steps, each after the
lengths are restored (events cannot be recorded inside a captured graph on
the runtime PyTorch ships). Also reported: per-step median and spread,
repeated timed runs, the unfused path (Shared stage + Non-Shared stage +
Merge) and the append alone, the Non-Shared stage's own HBM fraction, the
GPU's streaming-read bandwidth, the PagedAttention-style comparison, and the
fp64 oracle timed on the host's cores (a child process).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # fp32 vector

DEFAULT_CONFIG = "5"
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
    return int(s) if str(s).isdigit() else s


def algorithmic(w):
    """Algorithmic bytes / flops of one decode call on workload w."""
    e = w.elem_bytes
    # prompt rows once per distinct physical range (requests may alias one prefix)
    prompt_tokens = sum(p for (o, p) in {(int(w.prefix_off[r]), int(w.prefix_len[r])) for r in range(w.R)})
    gen_tokens = int(sum(w.B * int(w.unshared_len[r]) for r in range(w.R)))
    unique_kv = (prompt_tokens + gen_tokens) * w.Hkv * w.D * 2 * e
    q = w.N_b * w.Hq * w.D * e
    out = w.N_b * w.Hq * (w.D + 1) * 4
    slots = gen_tokens * 4
    total = unique_kv + q + out + slots
    mfma_flops = 4 * w.D * w.Hq * int(sum(w.B * int(w.prefix_len[r]) for r in range(w.R)))
    all_flops = 4 * w.D * w.Hq * int(sum(w.B * (int(w.prefix_len[r]) + int(w.unshared_len[r])) for r in range(w.R)))
    unshared = gen_tokens * w.Hkv * w.D * 2 * e + q + out + slots
    return dict(unique_kv=unique_kv, total=total, mfma_flops=mfma_flops, flops=all_flops,
                unshared_stage=unshared)


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
                  "generative_recommendation_beam_amd/csrc/valu_attn.hip",
                  "generative_recommendation_beam_amd/csrc/append.hip",
                  "generative_recommendation_beam_amd/csrc/merge.hip",
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


TRAFFIC_PATH = os.path.join(ROOT, "profiles", "traffic.json")


def measured_traffic(cfg, path=TRAFFIC_PATH):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    counts, each scaled by the same counter's reading for a plain copy of known
    size; None if absent or taken on different kernel sources."""
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    e = t.get("workloads", {}).get(str(cfg))
    if not e or e.get("kernel_hash") != kernel_hash():
        return None
    cal = t["copy_calibration"]
    return int(e["fetch_kib"] * 1024 * cal["fetch_factor"] + e["write_kib"] * 1024 * cal["write_factor"])


TRAFFIC_WORKLOADS = ("5", "2", "3", "4A", "4B")


def collect_traffic(d, path=TRAFFIC_PATH):
    """Write `path` (profiles/traffic.json) from rocprofv3 counter runs under directory
    d (host only, no GPU): d/copy_fetch and d/copy_write hold FETCH_SIZE and
    WRITE_SIZE of `bench.py --calibrate-copy 1073741824`; d/fetch_<cfg> and
    d/write_<cfg> those of `bench.py --config <cfg> --profile-steps 3`, with
    that run's stdout in d/fetch_<cfg>.log (its JSON line names the layers and
    the kernel sources). Each was written by
    rocprofv3 --pmc <COUNTER> --output-format csv -d d/<name> -o p -- python3 bench.py ..."""
    import csv

    def rows(name, ctr):
        fn = os.path.join(d, name, "p_counter_collection.csv")
        rs = [r for r in csv.DictReader(open(fn)) if r["Counter_Name"] == ctr]
        return sorted(rs, key=lambda r: int(r["Dispatch_Id"]))

    def copy_kib(name, ctr):
        rs = rows(name, ctr)
        cp = [r for r in rs if "copy" in r["Kernel_Name"].lower()] or rs[-1:]
        return float(cp[-1]["Counter_Value"])

    def run_info(name):
        for line in open(os.path.join(d, name + ".log")):
            if line.startswith("{") and "profile_steps" in line:
                return json.loads(line)
        raise SystemExit(f"collect_traffic: no profile-steps line in {name}.log")

    def per_call(name, ctr, n_layers):
        rs = rows(name, ctr)
        first = next(i for i, r in enumerate(rs) if "beam_topk" in r["Kernel_Name"])
        steps, cur = [], None
        for r in rs[first:]:
            if "beam_topk" in r["Kernel_Name"]:
                cur = []
                steps.append(cur)
            else:
                cur.append(float(r["Counter_Value"]))
        n_calls = len(steps) * n_layers
        return sum(map(sum, steps)) / n_calls, len(steps[-1]) // n_layers, n_calls

    cal_bytes = 1073741824
    fetch_c, write_c = copy_kib("copy_fetch", "FETCH_SIZE"), copy_kib("copy_write", "WRITE_SIZE")
    cal = dict(bytes=cal_bytes, fetch_kib=round(fetch_c, 3), write_kib=round(write_c, 3),
               fetch_factor=round(cal_bytes / 1024 / fetch_c, 4), write_factor=round(cal_bytes / 1024 / write_c, 4))
    out = {"about": ("HBM bytes per xattn_append_decode call (every kernel launch of the call) from rocprofv3 "
                     "--pmc FETCH_SIZE and WRITE_SIZE (KiB per dispatch, summed over the call's dispatches), "
                     "each scaled by the factor the same counter needs for a plain 1 GiB device-to-device copy "
                     "(bench.py --calibrate-copy 1073741824). Commands: rocprofv3 --pmc FETCH_SIZE (then "
                     "WRITE_SIZE) --output-format csv -d <dir> -o p -- python3 bench.py --config <cfg> "
                     "--profile-steps 3; the calls are the dispatches after the first beam selection (3 steps x "
                     "n_layers calls); written by bench.py --collect-traffic <dir>. kernel_hash identifies the "
                     "library sources the counts were taken on (bench.py kernel_hash()): the Shared-stage, "
                     "vector, append and merge kernels and the dispatch."),
           "copy_calibration": cal, "workloads": {}}
    for c in TRAFFIC_WORKLOADS:
        if not os.path.exists(os.path.join(d, f"fetch_{c}")):
            continue
        info = run_info(f"fetch_{c}")
        f, n_disp, n_calls = per_call(f"fetch_{c}", "FETCH_SIZE", info["n_layers"])
        w, _, _ = per_call(f"write_{c}", "WRITE_SIZE", info["n_layers"])
        out["workloads"][c] = dict(kernel_hash=info["kernel_hash"], fetch_kib=round(f, 2), write_kib=round(w, 2),
                                   dispatches_per_call=n_disp, calls=n_calls,
                                   traffic_bytes=int(f * 1024 * cal["fetch_factor"] + w * 1024 * cal["write_factor"]))
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out["workloads"]))


def _spread(xs):
    xs = list(xs)
    return dict(median=round(statistics.median(xs), 5), min=round(min(xs), 5), max=round(max(xs), 5),
                stdev=round(statistics.pstdev(xs), 5), n=len(xs))


class Setup:
    """One workload's n_layers resident on the device, with its step graph."""

    def __init__(self, cfg, n_layers, args):
        import torch
        from generative_recommendation_beam_amd import device as dv
        from generative_recommendation_beam_amd import inputs, xattn
        self.cfg, self.n_layers, self.args = cfg, n_layers, args
        self.layers_np = [inputs.config(cfg, layer=l) for l in range(n_layers)]
        w0 = self.w0 = self.layers_np[0]
        # One [n_layers][R] length array, restored with one copy per step.
        self.ulen_all = torch.zeros((n_layers, max(w0.R, 1)), dtype=torch.int32, device="cuda")
        self.layers = []
        for l, w in enumerate(self.layers_np):
            d = dv.upload(w, prefix_splits=args.prefix_splits, unshared_splits=args.unshared_splits,
                          rows_per_block=args.rows_per_block,
                          pipeline_stages=args.stages, key_groups=args.key_groups)
            d.unshared_len = self.ulen_all[l]
            table_in, table_out, t_last = dv.prepare_step(d)
            o, lse, ws, nb = dv.alloc_outputs(d, 3 if t_last is not None else 2)
            self.layers.append((d, o, lse, ws, nb, table_in, table_out, t_last))
        self.ulen0 = self.ulen_all.clone()
        # The step opens with the survivor selection (beam width x top-k pool
        # per request, top-k = beam width) whose parents every layer's append reads.
        self.topk_k = max(1, min(w0.B, 512))
        tx = inputs.make_topk("select", R=w0.R, BW=w0.B, K=self.topk_k, n_out=w0.B, seed_key=(700, 0))
        self.sel_in = [torch.from_numpy(v).cuda() for v in (tx.beam_score, tx.logprob, tx.token)]
        self.sel_parent = torch.empty((w0.R, w0.B), dtype=torch.int32, device="cuda")
        self.sel_tok = torch.empty_like(self.sel_parent)
        self.sel_score = torch.empty((w0.R, w0.B), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        self.plan = xattn.get_plan(self.layers[0][0].dims, 2)
        self.graphs = None
        if not args.eager:
            steps = []
            for (d, o, lse, ws, nb, tin, tout, t_last) in self.layers:
                st = dv.layer_step(d, o, lse, ws, nb, tin, tout, t_last)
                st.parent = self.sel_parent.data_ptr()
                steps.append(st)
            sel = lambda: xattn.beam_select(*self.sel_in, w0.B, self.sel_parent, self.sel_tok, self.sel_score)
            # the step; each layer's call alone, back to back (to time the
            # dominant kernel with HIP events around its launches); the plain
            # decodes on the complete caches; the selection alone
            self.graphs = dict(
                step=xattn.StepGraph(steps, select=sel()),
                layer=xattn.StepGraph(steps),
                decode=xattn.StepGraph([dv.layer_step(d, o, lse, ws, nb, None, tout, None)
                                        for (d, o, lse, ws, nb, tin, tout, t_last) in self.layers]),
                select=xattn.StepGraph([], select=sel()))
            torch.cuda.synchronize()

    def eager_step(self, evs=None):
        from generative_recommendation_beam_amd import xattn
        self.ulen_all.copy_(self.ulen0)
        xattn.beam_topk(*self.sel_in, self.w0.B, self.sel_parent, self.sel_tok, self.sel_score)
        for i, (d, o, lse, ws, nb, tin, tout, t_last) in enumerate(self.layers):
            if evs is not None:
                evs[i][0].record()
            if t_last is not None:
                xattn.append_decode(d.dims, q=d.q, k_shared=d.k_shared, v_shared=d.v_shared,
                                    prefix_off=d.prefix_off, prefix_len=d.prefix_len, k_new=d.k_new[t_last],
                                    v_new=d.v_new[t_last], parent=self.sel_parent, slot_base=d.slot_base,
                                    active=d.active[t_last], k_pool=d.k_pool, v_pool=d.v_pool, table_in=tin,
                                    table_out=tout, unshared_len=d.unshared_len, o=o, lse=lse,
                                    workspace=ws if nb else None, workspace_bytes=nb)
            else:
                xattn.decode(d.dims, d.q, d.k_shared, d.v_shared, d.prefix_off, d.prefix_len, d.k_pool,
                             d.v_pool, tout, d.unshared_len, o, lse, ws if nb else None, nb)
            if evs is not None:
                evs[i][1].record()

    def one_step(self, evs=None):
        if self.graphs is None:
            self.eager_step(evs)
        else:
            self.ulen_all.copy_(self.ulen0)
            self.graphs["step"].launch()

    def close(self):
        if self.graphs:
            for g in self.graphs.values():
                g.close()
        self.graphs = None


def _ev():
    import torch
    return torch.cuda.Event(enable_timing=True)


def time_steps(s, K, warmup, repeats, min_warm_s=0.0):
    """K timed steps after `warmup` untimed ones (more, until `min_warm_s`
    seconds of them have run: a workload measured right after another one
    finds the clocks where that one left them), bracketed by synchronizes,
    with one event pair around the whole run (events between the steps add
    their own gaps); then K more steps with an event pair around each step
    (and each call, eagerly) give the per-step median and spread, and
    `repeats` more timed runs of K steps the run-to-run spread."""
    import torch
    tw = time.perf_counter()
    n_warm = 0
    while n_warm < warmup or time.perf_counter() - tw < min_warm_s:
        s.one_step()
        n_warm += 1
        if n_warm >= warmup:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    start, end = _ev(), _ev()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for k in range(K):
        s.one_step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(end)
    per_step = [(_ev(), _ev()) for _ in range(K)]
    call_evs = [[(_ev(), _ev()) for _ in s.layers] for _ in range(K)] if s.graphs is None else None
    torch.cuda.synchronize()
    for k in range(K):
        per_step[k][0].record()
        s.one_step(None if call_evs is None else call_evs[k])
        per_step[k][1].record()
    torch.cuda.synchronize()
    step_ms = [a.elapsed_time(b) for a, b in per_step]
    reps = []
    for _ in range(repeats):
        a, b = _ev(), _ev()
        torch.cuda.synchronize()
        a.record()
        for k in range(K):
            s.one_step()
        b.record()
        torch.cuda.synchronize()
        reps.append(a.elapsed_time(b) / K)
    call_us = None
    if call_evs is not None:
        call_us = [a.elapsed_time(b) * 1e3 for evs in call_evs for a, b in evs]
    return dict(ms_total=ms_total, wall=wall, step_ms=step_ms, repeat_ms_per_step=reps, eager_call_us=call_us,
                warmup_steps=n_warm)


def time_graph(g, K, before=None):
    """Mean and per-launch ms of K launches of graph g, each between two HIP
    events on the launch stream (`before` runs outside the events)."""
    import torch
    pairs = [(_ev(), _ev()) for _ in range(K)]
    for e0, e1 in pairs:
        if before is not None:
            before()
        e0.record()
        g.launch()
        e1.record()
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in pairs]


def time_parts(s, K):
    """The same layers through the separate calls. Each kind of call is
    captured as one graph of the n_layers calls (torch's graph capture of the
    library's launches on the capture stream) and timed like the fused call,
    K launches between HIP events, interval / n_layers: the unfused path
    (Shared stage, Non-Shared stage, Merge) on the complete caches, and the
    append alone (lengths restored before each launch, outside the events)."""
    import numpy as np
    import torch
    from generative_recommendation_beam_amd import xattn
    bufs = []
    for (d, o, lse, ws, nb, tin, tout, t_last) in s.layers:
        rows, D = d.rows, d.w.D
        n0 = xattn.workspace_size(d.dims, 0)
        n1 = xattn.workspace_size(d.dims, 1)
        bufs.append(dict(os=torch.empty((rows, D), dtype=torch.float32, device="cuda"),
                         ls=torch.empty(rows, dtype=torch.float32, device="cuda"),
                         ou=torch.empty((rows, D), dtype=torch.float32, device="cuda"),
                         lu=torch.empty(rows, dtype=torch.float32, device="cuda"),
                         w0=torch.zeros(max(n0, 1), dtype=torch.uint8, device="cuda"), n0=n0,
                         w1=torch.zeros(max(n1, 1), dtype=torch.uint8, device="cuda"), n1=n1,
                         tscratch=torch.empty_like(tout)))
    layers = list(zip(s.layers, bufs))

    def shared():
        for (d, o, lse, ws, nb, tin, tout, t_last), b in layers:
            xattn.shared_stage(d.dims, d.q, d.k_shared, d.v_shared, d.prefix_off, d.prefix_len, b["os"], b["ls"],
                               b["w0"] if b["n0"] else None, b["n0"])

    def unshared():
        for (d, o, lse, ws, nb, tin, tout, t_last), b in layers:
            xattn.unshared_stage(d.dims, d.q, d.k_pool, d.v_pool, tout, d.unshared_len, b["ou"], b["lu"],
                                 b["w1"] if b["n1"] else None, b["n1"])

    def merge():
        for (d, o, lse, ws, nb, tin, tout, t_last), b in layers:
            xattn.merge(d.rows, d.w.D, b["os"], b["ls"], b["ou"], b["lu"], o, lse)

    def appends():
        for (d, o, lse, ws, nb, tin, tout, t_last), b in layers:
            xattn.cache_append(d.dims, d.k_new[t_last], d.v_new[t_last], s.sel_parent, d.slot_base,
                               d.active[t_last], d.k_pool, d.v_pool, tin, b["tscratch"], d.unshared_len)

    class _Replay:
        def __init__(self, fn):
            fn()  # eager warm-up
            torch.cuda.synchronize()
            self.g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(self.g):
                fn()
            torch.cuda.synchronize()

        def launch(self):
            self.g.replay()

    n = len(s.layers)
    per_call = lambda ms: round(float(np.median(ms)) * 1e3 / n, 3)
    # complete caches: lengths as after the step
    s.one_step()
    torch.cuda.synchronize()
    out = dict(shared_us=per_call(time_graph(_Replay(shared), K)),
               unshared_us=per_call(time_graph(_Replay(unshared), K)),
               merge_us=per_call(time_graph(_Replay(merge), K)))
    out["unfused_us"] = round(out["shared_us"] + out["unshared_us"] + out["merge_us"], 3)
    if s.layers[0][7] is not None:
        restore = lambda: s.ulen_all.copy_(s.ulen0)
        restore()
        g = _Replay(appends)
        out["append_us"] = per_call(time_graph(g, K, restore))
    out["timing"] = "each kind of call captured as one graph of the n_layers calls, K launches, interval / n_layers"
    # leave the caches as a step leaves them
    s.one_step()
    torch.cuda.synchronize()
    return out


def stream_bandwidth(nbytes=4 << 30, reps=10):
    """GB/s of the library's streaming-read kernel over nbytes of HBM."""
    import torch
    from generative_recommendation_beam_amd import xattn
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for _ in range(2):
        xattn.stream_read(buf, sink)
    ms = []
    for _ in range(reps):
        a, b = _ev(), _ev()
        a.record()
        xattn.stream_read(buf, sink)
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    del buf
    med = statistics.median(ms)
    return dict(read_GBps=round(nbytes / (med * 1e-3) / 1e9, 1), bytes=nbytes, reps=reps,
                frac_of_peak=round(nbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                kernel="xattn_stream_read (16-byte non-temporal loads, data discarded), median of the launches")


def cpu_baseline(cfg, seconds, single_core, single_seconds):
    """The fp64 oracle as it stands, timed on this host's cores in a child
    process (BLAS pinned to one thread per process before numpy loads)."""
    cmd = [sys.executable, "-m", "oracle.timing", "--config", str(cfg), "--seconds", str(seconds),
           "--single-core", ",".join(single_core), "--single-seconds", str(single_seconds)]
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=1200)
    if r.returncode != 0:
        raise RuntimeError(f"oracle timing failed ({r.returncode}):\n{r.stderr[-2000:]}")
    return json.loads(r.stdout.strip().splitlines()[-1])


def paged_baseline(s, K, xattn_decode_us, xattn_call_us, xattn_step_ms):
    """The same layers in a PagedAttention-style block-paged cache: per layer,
    the copies branching beams make of their partial tail blocks, then the
    per-beam paged decode. HIP events around every call, K rounds, queued
    behind each other (each call outlasts its host launch)."""
    import numpy as np
    import torch
    from generative_recommendation_beam_amd import device as dv
    from generative_recommendation_beam_amd import xattn
    paged = []
    for (d, o, lse, ws, nb, tin, tout, t_last) in s.layers:
        pc = dv.build_paged(d, tout)
        pnb = xattn.paged_workspace_size(d.dims, pc.max_seq_len)
        pws = torch.zeros(max(pnb, 1), dtype=torch.uint8, device="cuda")
        paged.append((d, pc, o, lse, pws, pnb))
    torch.cuda.synchronize()
    rounds = [[(_ev(), _ev(), _ev()) for _ in paged] for _ in range(K)]
    for d, pc, o, lse, pws, pnb in paged:  # warm-up
        xattn.paged_copy_blocks(d.dims, pc.k_cache, pc.v_cache, pc.parent_tail, pc.spare)
        dv.paged_decode(d, pc, o, lse, pws, pnb)
    torch.cuda.synchronize()
    start, end = _ev(), _ev()
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
    step_ms = start.elapsed_time(end) / K  # every layer's copies and decode
    pc0 = paged[0][1]
    del paged
    torch.cuda.empty_cache()
    return dict(decode_us_per_call=round(dec_us, 2), block_copy_us_per_call=round(copy_us, 2),
                step_ms=round(step_ms, 4), blocks_per_layer=int(pc0.k_cache.shape[0]), rounds=K,
                decode_speedup_xattn=round(dec_us / xattn_decode_us, 2),
                layer_speedup_xattn=round((copy_us + dec_us) / xattn_call_us, 2),
                step_speedup_xattn=round(step_ms / xattn_step_ms, 2),
                note="same layers, same attention; PagedAttention-style per-beam paged decode "
                     "(16-token blocks, prompt blocks shared and re-read by every beam) plus the "
                     "copy each beam makes of its parent's tail block; eager launches. "
                     "decode_speedup_xattn: against xattn's decode alone; layer_speedup_xattn: "
                     "copy + decode against the fused append + decode call; step_ms: every "
                     "layer's copies and decode, against xattn's whole step")


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


def measure(cfg, args, *, paged_rounds, min_warm_s=0.0):
    """Every GPU figure of one workload: the timed steps (value), the
    dominant kernel's roofline, the separate calls and the comparison."""
    import numpy as np
    import torch
    n_layers = args.layers or DEFAULT_LAYERS[str(cfg)]
    s = Setup(cfg, n_layers, args)
    w0, K = s.w0, args.steps
    print(f"[{cfg}] timing {K} steps of {n_layers} layers ...", file=sys.stderr, flush=True)
    st = time_steps(s, K, args.warmup, args.repeats, min_warm_s)
    ms_per_step = st["ms_total"] / K
    value = w0.N_b * n_layers / (ms_per_step / 1e3)
    restore = lambda: s.ulen_all.copy_(s.ulen0)  # the same append every launch
    if s.graphs is None:
        call_us = float(np.mean(st["eager_call_us"]))
        decode_only_us = select_us = None
    else:
        call_us = float(np.mean(time_graph(s.graphs["layer"], K, restore))) * 1e3 / n_layers
        decode_only_us = float(np.mean(time_graph(s.graphs["decode"], K))) * 1e3 / n_layers
        select_us = float(np.mean(time_graph(s.graphs["select"], K))) * 1e3
    alg = algorithmic(w0)
    appends = s.layers[0][7] is not None
    fused = appends and s.plan["mfma"] == 1 and s.plan["partials"] == 0
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
    folded_prompt = appends and s.plan["mfma"] == 1 and s.plan["partials"] > 0 and s.plan["unshared_splits"] > 0
    if fused:
        roof["kernel"] = "xattn_append_decode call (1 kernel launch: the append folded into the decode)"
    elif folded_prompt:
        roof["kernel"] = ("xattn_append_decode call (%d kernel launches: the prompt pass with the append folded "
                          "in, then the Non-Shared pass%s)" % (
                              s.plan["launches"], " folding the prompt's partials in" if s.plan["launches"] == 2
                              else ", then the Merge"))
    elif appends:
        roof["kernel"] = "xattn_append_decode call (append, then %d decode launch%s)" % (
            s.plan["launches"], "" if s.plan["launches"] == 1 else "es")
    else:
        roof["kernel"] = "xattn_decode call (%d kernel launch%s)" % (
            s.plan["launches"], "" if s.plan["launches"] == 1 else "es")
    roof["timing"] = ("HIP events around K launches of a graph of the n_layers calls (interval / "
                      "n_layers; lengths restored before each launch, outside the events), run right "
                      "after the timed steps" if s.graphs is not None else
                      "HIP events around every call of the timed steps")
    roof["avg_call_us"] = round(call_us, 3)
    if decode_only_us is not None:
        roof["decode_only_us"] = round(decode_only_us, 3)
    roof["algorithmic_bytes_per_call"] = call_bytes
    roof["algorithmic_mfma_flops_per_call"] = alg["mfma_flops"]
    roof["hbm_frac_algorithmic"] = round(call_bytes / call_s / 1e9 / PEAK_HBM_GBS, 4)
    roof["mfma_frac_algorithmic"] = round(alg["mfma_flops"] / call_s / 1e12 / peak_tflops, 4)
    roof["kernel_hash"] = kernel_hash()
    print(f"[{cfg}] timing the separate calls ...", file=sys.stderr, flush=True)
    parts = time_parts(s, min(K, 20))
    ns_s = parts["unshared_us"] * 1e-6
    parts["nonshared_stage"] = dict(
        us=parts["unshared_us"], algorithmic_bytes=alg["unshared_stage"],
        achieved_GBps=round(alg["unshared_stage"] / ns_s / 1e9, 1),
        frac_of_hbm_peak=round(alg["unshared_stage"] / ns_s / 1e9 / PEAK_HBM_GBS, 4),
        bytes="generated K/V once per beam + Q + O + lse + slot indices")
    parts["unfused_vs_fused"] = round(parts["unfused_us"] / (decode_only_us or call_us), 3)
    res = {
        "value": round(value, 1),
        "ms_per_step": round(ms_per_step, 5),
        "step_ms_spread": _spread(st["step_ms"]),
        "repeat_ms_per_step": [round(x, 5) for x in st["repeat_ms_per_step"]],
        "warmup_steps": st["warmup_steps"],
        "wall_s_timed": round(st["wall"], 4),
        "config": {"workload": WORKLOAD_NAMES[str(cfg)], "n_layers": n_layers, "beams_per_call": w0.N_b,
                   "step": "beam selection (%d x %d x %d pool -> %d beams per request), then "
                           "append + decode per layer (one xattn_append_decode call)" % (
                               w0.R, w0.B, s.topk_k, w0.B),
                   "launch": "eager" if s.graphs is None else "graph", "plan": s.plan},
        "dtype": w0.dtype,
        "unique_kv_GBps": round(alg["unique_kv"] / call_s / 1e9, 1),
        "total_GBps": round(call_bytes / call_s / 1e9, 1),
        "mfma_TFLOPs": round(alg["mfma_flops"] / call_s / 1e12, 1),
        "step_GBps": round(n_layers * call_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "roofline": roof,
        "beam_select_us": None if select_us is None else round(select_us, 3),
        "separate_calls": parts,
    }
    if paged_rounds and w0.dtype == "bf16":
        print(f"[{cfg}] timing the PagedAttention-style baseline ...", file=sys.stderr, flush=True)
        res["paged_baseline"] = paged_baseline(s, paged_rounds, decode_only_us or call_us, call_us, ms_per_step)
    s.close()
    del s
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--repeats", type=int, default=2, help="extra timed runs of K steps (run-to-run spread)")
    ap.add_argument("--config", default=DEFAULT_CONFIG)
    ap.add_argument("--extra-configs", default=None,
                    help="comma list measured after the headline (default: 2 with the default headline)")
    ap.add_argument("--layers", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--prefix-splits", type=int, default=0, help="override the split plan (0 = auto)")
    ap.add_argument("--unshared-splits", type=int, default=0,
                    help="override the generated-token splits (0 = auto)")
    ap.add_argument("--rows-per-block", type=int, default=0, help="override rows per workgroup (0 = auto)")
    ap.add_argument("--stages", type=int, default=0, help="override LDS pipeline stages (0 = auto)")
    ap.add_argument("--key-groups", type=int, default=0, help="override key groups per workgroup (0 = auto)")
    ap.add_argument("--no-paged", action="store_true",
                    help="skip the PagedAttention-style baseline measured beside the step")
    ap.add_argument("--no-stream", action="store_true", help="skip the streaming-read bandwidth")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run one plain device-to-device copy of BYTES (the reference kernel "
                         "the HBM byte counters are scaled by) and exit")
    ap.add_argument("--profile-steps", type=int, default=0, metavar="N",
                    help="only build the workload and run N eager steps (for counter collection), then exit")
    ap.add_argument("--eager", action="store_true",
                    help="launch every call from the host instead of one captured step graph")
    ap.add_argument("--collect-traffic", default=None, metavar="DIR",
                    help="host only: write profiles/traffic.json from the rocprofv3 counter runs under DIR, then exit")
    args = ap.parse_args()
    if args.collect_traffic:
        collect_traffic(args.collect_traffic)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(whole requests would be placed per GPU, with no exchange inside attention).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from generative_recommendation_beam_amd import xattn

    if not os.path.exists(xattn.LIB_PATH):
        raise SystemExit(f"bench.py: {xattn.LIB_PATH} is not built (run __graft_entry__.build())")
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        n = args.calibrate_copy // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n * 4}), flush=True)
        return
    cfg = _cfg_key(args.config)
    if args.profile_steps:
        # Counter collection: the workload's calls only, eagerly (every
        # dispatch after the first beam selection belongs to a step).
        args.eager = True
        s = Setup(cfg, args.layers or DEFAULT_LAYERS[str(cfg)], args)
        for _ in range(args.profile_steps):
            s.one_step()
        torch.cuda.synchronize()
        print(json.dumps({"profile_steps": args.profile_steps, "config": WORKLOAD_NAMES[str(cfg)],
                          "n_layers": s.n_layers, "plan": s.plan, "kernel_hash": kernel_hash()}), flush=True)
        s.close()
        return
    extras = args.extra_configs
    if extras is None:
        extras = "2" if str(cfg) == DEFAULT_CONFIG else ""
    extras = [_cfg_key(c) for c in extras.split(",") if c]

    head = measure(cfg, args, paged_rounds=0 if args.no_paged else min(args.steps, 5))
    result = {
        "metric": "beam-decode attention beams*layer-steps/s; achieved HBM GB/s vs peak",
        "value": head.pop("value"),
        "unit": "beams*layer-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head.pop("dtype"),
        "data": "synthetic",
        "config": head.pop("config"),
    }
    result.update(head)
    for c in extras:
        ex = measure(c, args, paged_rounds=0 if args.no_paged else min(args.steps, 20), min_warm_s=0.05)
        result[f"config_{c}"] = ex
    if not args.no_stream:
        result["hbm_stream_read"] = stream_bandwidth()
    result["batch_former"] = batch_former_timing()
    if not args.no_cpu_baseline:
        print("timing the oracle on host cores (child process) ...", file=sys.stderr, flush=True)
        cb = cpu_baseline(cfg, args.cpu_seconds, ["1", "2", "4A"], 5.0)
        result["cpu_baseline"] = cb["multi"]
        result["cpu_baseline_single_core"] = cb["single_core"]
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
