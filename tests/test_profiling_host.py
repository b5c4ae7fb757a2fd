"""The rocprofv3 summary helpers on hand-made CSV files: calibrated HBM bytes per
dispatch and per step, the source-hash guard, and the in-step span of kernels
launched in pairs."""
import csv
import os

import pytest

from precision_moe_amd import profiling as prof


def _counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (k, c, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def _trace(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_kernel_trace.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for k, a, b in rows:
            w.writerow({"Kernel_Name": k, "Start_Timestamp": a, "End_Timestamp": b})


K1 = "void pmoe::fc_half_kernel<1, 0>(pmoe::FcParams)"


def test_traffic_per_dispatch_and_per_step(tmp_path):
    t = str(tmp_path)
    copy = 1 << 30
    # the copy kernel: FETCH_SIZE reads half the bytes (factor 2), WRITE_SIZE all of them
    _counters(f"{t}/cf", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", copy / 2048)])
    _counters(f"{t}/cw", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", copy / 1024)])
    # two dispatches per step of different size (the two parts of the experts)
    _counters(f"{t}/f", [(K1, "FETCH_SIZE", 400.0), (K1, "FETCH_SIZE", 600.0), ("other", "FETCH_SIZE", 9.0)])
    _counters(f"{t}/w", [(K1, "WRITE_SIZE", 10.0), (K1, "WRITE_SIZE", 30.0)])
    out = f"{t}/traffic.txt"
    prof.write_traffic(f"{t}/f", f"{t}/w", f"{t}/cf", f"{t}/cw", copy, "fc_half_kernel<1, 0>",
                       "wl", out, "cmd", launches=2)
    per_dispatch = (500.0 * 2 + 20.0) * 1024
    kv = dict(l.strip().split("=", 1) for l in open(out) if "=" in l and not l.startswith("#"))
    assert float(kv["hbm_bytes_per_dispatch"]) == pytest.approx(per_dispatch, rel=1e-6)
    assert float(kv["hbm_bytes_per_step"]) == pytest.approx(2 * per_dispatch, rel=1e-6)
    assert prof.read_traffic(out, "wl") == pytest.approx(2 * per_dispatch, rel=1e-6)
    assert prof.read_traffic(out, "another_workload") is None
    # measured with other GEMM sources: not reported
    text = open(out).read().replace(f"source_sha256={prof.gemm_source_hash()}", "source_sha256=0")
    open(out, "w").write(text)
    assert prof.read_traffic(out, "wl") is None
    assert prof.read_traffic(f"{t}/missing.txt", "wl") is None


def test_in_step_spans_of_paired_launches(tmp_path):
    t = str(tmp_path)
    # three steps; each runs the kernel twice, overlapping, on two streams
    us = 1000  # timestamps are in ns
    rows = [(K1, 100 * us, 600 * us), (K1, 110 * us, 800 * us),
            (K1, 2000 * us, 2500 * us), (K1, 2010 * us, 2650 * us),
            (K1, 4000 * us, 4400 * us), (K1, 4005 * us, 4700 * us)]
    _trace(f"{t}/kt", rows + [("void pmoe::finalize_kernel(int)", 900 * us, 950 * us)])
    times = prof.dispatch_times(f"{t}/kt", "pmoe::fc_half_kernel<1, 0>")
    assert len(times) == 6
    assert prof.pair_spans(times) == [700.0, 650.0, 700.0]
    out = f"{t}/spans.txt"
    prof.write_spans(f"{t}/kt", "wl", out, "cmd", "pmoe::fc_half_kernel<1, 0>", 1, 2)
    kv = dict(l.strip().split("=", 1) for l in open(out) if "=" in l and not l.startswith("#"))
    assert kv["pairs"] == "3" and kv["pairs_selected"] == "1..2"
    assert float(kv["avg_span_us_selected"]) == pytest.approx(675.0)
