"""Host logic of the rocprofv3 summariser (CPU): counter scaling by the copy
calibration, per-call sums over a workload's kernels, the per-XCD MFMA busy
share, and the source hash that bench.py checks."""
import csv
import json
import os

import bench
from retention_chunkwise_amd import profsum as P

HDR = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(HDR)
        w.writerows(rows)


def _kernels():
    names = [k for spec in P.WORKLOADS.values() for k, _ in spec["kernels"]]
    return sorted(set(names))


def test_traffic_scales_by_the_copy_and_sums_a_call(tmp_path):
    ks = _kernels()
    # the copy reads back half its bytes on FETCH_SIZE and all of them on WRITE_SIZE
    f_rows = [[1, P.COPY_KERNEL + "(void*)", "FETCH_SIZE", (1 << 20) / 2]]
    w_rows = [[1, P.COPY_KERNEL + "(void*)", "WRITE_SIZE", 1 << 20]]
    for i, k in enumerate(ks):
        name = "void ret::" + k.lstrip(":") + "(ret::Args)"
        # two dispatches of each kernel, the counter split over two instances each
        for d in (10 + 2 * i, 11 + 2 * i):
            f_rows += [[d, name, "FETCH_SIZE", 300.0], [d, name, "FETCH_SIZE", 200.0]]
            w_rows += [[d, name, "WRITE_SIZE", 100.0]]
    _csv(tmp_path / "f.csv", f_rows)
    _csv(tmp_path / "w.csv", w_rows)
    P.traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), out_dir=str(tmp_path))
    d = json.load(open(tmp_path / "hbm_traffic_fwd_ret_fwd_long_bf16.json"))
    assert abs(d["fetch_scale"] - 2.0) < 1e-12 and abs(d["write_scale"] - 1.0) < 1e-12
    # two kernels per call, 500 KiB fetched (x2) and 100 KiB written per dispatch
    assert abs(d["bytes_per_launch"] - 2 * (500 * 1024 * 2 + 100 * 1024)) < 1e-6
    assert d["source_sha"] == bench.sources_sha(bench.FWD_SOURCES)
    b = json.load(open(tmp_path / "hbm_traffic_bwd_ret_fwd_long_bf16.json"))
    # the backward: two state passes, the fused reverse walk and the dq walk, 4 dispatches per call
    assert abs(b["bytes_per_launch"] - 4 * (500 * 1024 * 2 + 100 * 1024)) < 1e-6


def test_mfma_busy_uses_one_xcd_of_active_cycles(tmp_path):
    walk = "void ret::seg::seg_walk_kernel<128, 128, 128, 0>(ret::SegArgs)"
    state = "void ret::seg::seg_state_kernel<128, 128, 0, false>(ret::SegArgs)"
    act = 1000.0  # active cycles of one XCD
    rows = []
    for d, name, busy_frac, mops in ((1, walk, 0.25, 4.0e8), (2, state, 0.125, 1.0e8)):
        rows += [[d, name, "GRBM_GUI_ACTIVE", act * P.XCDS],
                 [d, name, "SQ_VALU_MFMA_BUSY_CYCLES", busy_frac * act * P.SIMDS],
                 [d, name, "SQ_INSTS_VALU_MFMA_MOPS_BF16", mops],
                 [d, name, "SQ_INSTS_VALU_MFMA_MOPS_F32", 0.0]]
    _csv(tmp_path / "m.csv", rows)
    with open(tmp_path / "s.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow([walk, 1, 400000, 400000, 50, 400000, 400000, 0])
        w.writerow([state, 1, 200000, 200000, 50, 200000, 200000, 0])
    P.mfma(str(tmp_path / "m.csv"), str(tmp_path / "s.csv"), out_dir=str(tmp_path))
    d = json.load(open(tmp_path / "mfma_fwd_ret_fwd_long_bf16.json"))
    assert abs(d["walk"]["mfma_busy"] - 0.25) < 1e-12 and abs(d["state"]["mfma_busy"] - 0.125) < 1e-12
    assert d["issued_bf16_flops_per_call"] == 5.0e8 * 512
    assert d["source_sha"] == bench.sources_sha(bench.FWD_SOURCES)
    md = open(tmp_path / "mfma_bench_workloads.md").read()
    # 4e8 x 512 FLOPs in 400 us = 512 TFLOP/s, 20.5 % of the bf16 peak
    assert "25.0 %" in md and "512.0 (bf16)" in md and "20.5 %" in md


def test_bench_ignores_summaries_of_other_sources(tmp_path, monkeypatch):
    p = tmp_path / "hbm_traffic_x.json"
    p.write_text(json.dumps({"source_sha": "0" * 16, "bytes_per_launch": 1.0}))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.measured_traffic("x", bench.FWD_SOURCES) is None
    p.write_text(json.dumps({"source_sha": bench.sources_sha(bench.FWD_SOURCES), "bytes_per_launch": 1.0}))
    assert bench.measured_traffic("x", bench.FWD_SOURCES)["bytes_per_launch"] == 1.0
