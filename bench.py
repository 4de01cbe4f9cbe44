"""Benchmark: staged beam-search decode attention on one MI355X.

One step = one decode step of every layer: ``xattn_decode`` on n_layers
distinct layer buffers (distinct Q, prompt KV, Non-Shared pool and slot table
per layer, so the working set defeats the 256 MB Infinity Cache), on
synthetic inputs shaped like the GR semantic-ID workload by default (8
requests, 1024-token user-history prompt, beam width 128, 3 generated tokens,
16 q / 4 kv heads, head dim 128, bf16). Inputs are resident in HBM before the
timed region; appends that build the Non-Shared cache happen before it.

Prints ONE JSON line. Metric: beams * layer-steps per second, plus achieved
HBM bandwidth on algorithmic bytes (unique KV: prompt KV once per request,
generated KV once per beam) and the roofline of the dominant kernel.
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

DEFAULT_LAYERS = {"1": 1, "2": 16, "3": 6, "4A": 3, "4B": 2, "5": 2}
WORKLOAD_NAMES = {
    "1": "tiny fp32: R=1 P=256 B=4 L=2 4q/1kv D=64",
    "2": "GR semantic-ID decode: R=8 P=1024 B=128 L=3 16q/4kv D=128 bf16",
    "3": "wide beam: R=4 P=2048 B=512 L=1-3 32q/8kv D=128 bf16",
    "4A": "prefix-homogeneous: 4 prefixes x 16 seqs P=4096 +512 unique, 32q/8kv D=128 bf16",
    "4B": "prefix-heterogeneous: 64 prefixes P=4096 +512 unique, 32q/8kv D=128 bf16",
    "5": "long history: R=16 P=16384 B=256 L=8 64q/8kv D=128 bf16",
}


def _cfg_key(s):
    return int(s) if s.isdigit() else s


def algorithmic(w):
    """Algorithmic bytes / flops of one decode call on workload w."""
    e = w.elem_bytes
    kv_tokens = int(sum(int(w.prefix_len[r]) + w.B * int(w.unshared_len[r]) for r in range(w.R)))
    unique_kv = kv_tokens * w.Hkv * w.D * 2 * e
    q = w.N_b * w.Hq * w.D * e
    out = w.N_b * w.Hq * (w.D + 1) * 4
    slots = int(sum(w.B * int(w.unshared_len[r]) for r in range(w.R))) * 4
    total = unique_kv + q + out + slots
    mfma_flops = 4 * w.D * w.Hq * int(sum(w.B * int(w.prefix_len[r]) for r in range(w.R)))
    all_flops = 4 * w.D * w.Hq * int(sum(w.B * (int(w.prefix_len[r]) + int(w.unshared_len[r])) for r in range(w.R)))
    return dict(unique_kv=unique_kv, total=total, mfma_flops=mfma_flops, flops=all_flops)


def cpu_baseline(layers_np, min_seconds=10.0):
    """Time the oracle (as it stands) on whole layers until min_seconds pass."""
    from oracle import pool
    done_beams = 0
    done_layers = 0
    t0 = time.perf_counter()
    workers = pool.host_cores()
    i = 0
    while True:
        w = layers_np[i % len(layers_np)]
        _, _, dt, used = pool.attention_parallel(w, workers=workers)
        done_beams += w.N_b
        done_layers += 1
        i += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    el = time.perf_counter() - t0
    return dict(value=done_beams / el, unit="beams*layer-steps/s", cores=used, kind="oracle",
                sample=f"{done_layers} full layer decode steps of the same workload "
                       f"(fp64 numpy oracle, {used} worker processes, {el:.1f} s)")


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
    layers = []
    for w in layers_np:
        d = dv.upload(w, prefix_splits=args.prefix_splits, rows_per_block=args.rows_per_block,
                      pipeline_stages=args.stages, key_groups=args.key_groups)
        dv.build_cache(d)
        o, lse, ws, nb = dv.alloc_outputs(d, 2)
        layers.append((d, o, lse, ws, nb))
    torch.cuda.synchronize()
    w0 = layers_np[0]
    plan = xattn.get_plan(layers[0][0].dims, 2)
    alg = algorithmic(w0)

    def one_step(evs=None):
        for i, (d, o, lse, ws, nb) in enumerate(layers):
            if evs is not None:
                evs[i][0].record()
            dv.decode(d, o, lse, ws, nb)
            if evs is not None:
                evs[i][1].record()

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()

    K = args.steps
    call_evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
                 for _ in layers] for _ in range(K)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for k in range(K):
        one_step(call_evs[k])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(end)
    call_ms = np.array([[e[0].elapsed_time(e[1]) for e in step] for step in call_evs])
    call_us = float(call_ms.mean() * 1e3)

    ms_per_step = ms_total / K
    value = w0.N_b * n_layers / (ms_per_step / 1e3)
    t_hbm = alg["total"] / (PEAK_HBM_GBS * 1e9)
    peak_tflops = PEAK_BF16_TFLOPS if w0.dtype == "bf16" else PEAK_FP32_TFLOPS
    t_mfma = alg["mfma_flops"] / (peak_tflops * 1e12)
    call_s = call_us * 1e-6
    if t_hbm >= t_mfma:
        achieved = alg["total"] / call_s / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(achieved / PEAK_HBM_GBS, 4), traffic=measured_traffic(cfg))
    else:
        achieved = alg["mfma_flops"] / call_s / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=peak_tflops, unit="TFLOP/s",
                    frac=round(achieved / peak_tflops, 4), traffic=measured_traffic(cfg))
    roof["kernel"] = "xattn_decode call (%d kernel launch%s)" % (plan["launches"], "" if plan["launches"] == 1 else "es")
    roof["avg_call_us"] = round(call_us, 3)
    roof["algorithmic_bytes_per_call"] = alg["total"]
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
                   "beams_per_call": w0.N_b, "plan": plan},
        "unique_kv_GBps": round(alg["unique_kv"] / call_s / 1e9, 1),
        "total_GBps": round(alg["total"] / call_s / 1e9, 1),
        "mfma_TFLOPs": round(alg["mfma_flops"] / call_s / 1e12, 1),
        "wall_s_timed": round(wall, 4),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print("timing the oracle on host cores ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(layers_np, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
