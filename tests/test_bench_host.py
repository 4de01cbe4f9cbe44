"""Host logic of bench.py (no GPU): the algorithmic byte and flop counts the
roofline divides by, and the HBM-traffic bookkeeping that turns rocprofv3
counter CSVs into profiles/traffic.json and back into roofline.traffic."""
import csv
import json
import types

import numpy as np
import pytest

import bench


def test_algorithmic_counts_aliased_prompt_once():
    # Two requests on one physical prompt range (offset 0, 10 tokens): the
    # prompt K/V counts once; generated tokens count once per beam.
    w = types.SimpleNamespace(elem_bytes=2, R=2, B=3, Hq=2, Hkv=1, D=4, N_b=6,
                              prefix_off=np.array([0, 0]), prefix_len=np.array([10, 10]),
                              unshared_len=np.array([2, 1]))
    a = bench.algorithmic(w)
    gen = 3 * 2 + 3 * 1                      # beams x generated tokens
    assert a["unique_kv"] == (10 + gen) * 1 * 4 * 2 * 2
    q, out, slots = 6 * 2 * 4 * 2, 6 * 2 * (4 + 1) * 4, gen * 4
    assert a["total"] == a["unique_kv"] + q + out + slots
    assert a["mfma_flops"] == 4 * 4 * 2 * (3 * 10 + 3 * 10)
    assert a["flops"] == 4 * 4 * 2 * (3 * 12 + 3 * 11)
    assert a["unshared_stage"] == gen * 1 * 4 * 2 * 2 + q + out + slots
    w.prefix_off = np.array([0, 10])         # disjoint ranges: both count
    assert bench.algorithmic(w)["unique_kv"] == (20 + gen) * 1 * 4 * 2 * 2


def _counters(path, rows, counter):
    path.mkdir()
    with open(path / "p_counter_collection.csv", "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for i, (name, value) in enumerate(rows):
            wr.writerow(dict(Dispatch_Id=i + 1, Kernel_Name=name, Counter_Name=counter, Counter_Value=value))


def _step_rows(per_call, n_layers, steps):
    rows = [("setup_fill_kernel", 999.0), ("append_kernel", 777.0)]  # before the first selection: ignored
    for _ in range(steps):
        rows.append(("xattn::beam_topk_kernel(xattn::TopkArgs)", 55.0))  # the selection itself: ignored
        for _ in range(n_layers):
            rows += [("shared_mfma_kernel<128, 8, 2, 4, false>", per_call[0]),
                     ("valu_attn_kernel<unsigned short, 128, 4, true, true>", per_call[1])]
    return rows


def test_collect_and_read_traffic(tmp_path):
    d = tmp_path / "prof"
    d.mkdir()
    # a 1 GiB copy reads as half its size on FETCH_SIZE, in full on WRITE_SIZE
    _counters(d / "copy_fetch", [("other", 1.0), ("__amd_rocclr_copyBuffer", 524288.0)], "FETCH_SIZE")
    _counters(d / "copy_write", [("__amd_rocclr_copyBuffer", 1048576.0)], "WRITE_SIZE")
    n_layers, steps = 3, 3
    _counters(d / "fetch_4A", _step_rows((100.0, 300.0), n_layers, steps), "FETCH_SIZE")
    _counters(d / "write_4A", _step_rows((10.0, 20.0), n_layers, steps), "WRITE_SIZE")
    h = bench.kernel_hash()
    (d / "fetch_4A.log").write_text("warming up\n" + json.dumps(
        {"profile_steps": steps, "n_layers": n_layers, "kernel_hash": h}) + "\n")
    out = tmp_path / "traffic.json"
    bench.collect_traffic(str(d), path=str(out))
    t = json.loads(out.read_text())
    assert t["copy_calibration"]["fetch_factor"] == 2.0 and t["copy_calibration"]["write_factor"] == 1.0
    e = t["workloads"]["4A"]
    assert set(t["workloads"]) == {"4A"}  # workloads without counter runs are left out
    assert e["fetch_kib"] == 400.0 and e["write_kib"] == 30.0
    assert e["dispatches_per_call"] == 2 and e["calls"] == steps * n_layers
    assert e["traffic_bytes"] == 400 * 1024 * 2 + 30 * 1024
    assert bench.measured_traffic("4A", path=str(out)) == e["traffic_bytes"]
    assert bench.measured_traffic("2", path=str(out)) is None       # not measured
    e["kernel_hash"] = "0" * 16
    out.write_text(json.dumps(t))
    assert bench.measured_traffic("4A", path=str(out)) is None      # other library sources
    assert bench.measured_traffic("4A", path=str(tmp_path / "absent.json")) is None


def test_committed_traffic_names_its_sources():
    t = json.load(open(bench.TRAFFIC_PATH))
    cal = t["copy_calibration"]
    assert cal["fetch_factor"] > 0 and cal["write_factor"] > 0
    for cfg, e in t["workloads"].items():
        assert cfg in bench.TRAFFIC_WORKLOADS and len(e["kernel_hash"]) == 16
        want = int(e["fetch_kib"] * 1024 * cal["fetch_factor"] + e["write_kib"] * 1024 * cal["write_factor"])
        # the KiB fields are stored to 0.01 KiB, the bytes from the unrounded means
        assert abs(e["traffic_bytes"] - want) <= 0.005 * 1024 * (cal["fetch_factor"] + cal["write_factor"])
