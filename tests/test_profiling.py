"""The profile summaries (kernel durations, calibrated HBM traffic, MFMA utilisation)
built from rocprofv3 CSV output, on small hand-made CSVs (CPU)."""

from __future__ import annotations

import csv
import json
import os

import pytest

from block_diffusion_sparse_herald_amd import profiling as P

ATTN = "void herald::attn_kernel<128>(unsigned short const*, float)"
COMBINE = "void herald::attn_combine_kernel<128>(unsigned short const*)"
SCAN = "void herald::scan_mfma_kernel<128>(unsigned short const*)"
COPY = "__amd_rocclr_copyBuffer"


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def _stats(d):
    _write(os.path.join(d, "run_kernel_stats.csv"), ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"],
           [[ATTN, 8, 7000.0, 6000.0, 9000.0, 40.0], [COMBINE, 8, 4000.0, 3000.0, 5000.0, 20.0],
            [SCAN, 1, 17000.0, 16000.0, 18000.0, 30.0]])


def _counters(d, counter, per_kernel):
    rows = []
    for name, grid, values in per_kernel:
        for v in values:
            rows.append([name, grid, counter, v])
    _write(os.path.join(d, "run_counter_collection.csv"), ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"],
           rows)


def test_traffic_calibrated_by_the_copy_kernel(tmp_path):
    st, fe, wr = (str(tmp_path / x) for x in ("stats", "fetch", "write"))
    _stats(st)
    copy_bytes = 64 << 20
    # the copy reads half of what it moves (the counter's unit), writes all of it
    _counters(fe, "FETCH_SIZE", [(COPY, 4096, [32768.0, 32768.0]), (COPY, 64, [1.0]), (ATTN, 512, [100.0, 300.0]),
                                 (COMBINE, 64, [50.0]), (SCAN, 1024, [1000.0])])
    _counters(wr, "WRITE_SIZE", [(COPY, 4096, [65536.0]), (ATTN, 512, [10.0, 30.0]), (COMBINE, 64, [5.0]),
                                 (SCAN, 1024, [40.0])])
    out = str(tmp_path / "out")
    assert P.main(["--workload", "w", "--stats", st, "--fetch", fe, "--write", wr, "--copy-bytes", str(copy_bytes),
                   "--out-dir", out]) == 0
    doc = json.load(open(os.path.join(out, "hbm_traffic_w.json")))
    cal = doc["calibration"]
    assert cal["fetch_factor"] == pytest.approx(2.0) and cal["write_factor"] == pytest.approx(1.0)
    by = {e["kernel"]: e for e in doc["entries"]}
    # mean per dispatch, both kernels of the attention call added, scaled to bytes
    assert by["attn_kernel+attn_combine_kernel"]["bytes_per_launch"] == round(((200.0 + 50.0) * 2.0 + (20.0 + 5.0)) * 1024)
    assert by["attn_kernel"]["bytes_per_launch"] == round((200.0 * 2.0 + 20.0) * 1024)
    assert by["scan"]["bytes_per_launch"] == round((1000.0 * 2.0 + 40.0) * 1024)
    assert by["scan"]["sources_sha256"] == P.sources_digest(P.KERNELS["scan"][1])
    md = open(os.path.join(out, "kernel_stats_w.md")).read()
    assert "| `herald::attn_kernel<128>` | 8 | 7.00 | 6.00 | 9.00 | 40.00 |" in md


def test_mfma_summary(tmp_path):
    st, mf = str(tmp_path / "stats"), str(tmp_path / "mfma")
    _stats(st)
    rows = []
    for v in (10.0, 12.0):
        rows.append([ATTN, 512, "MfmaUtil", v])
        rows.append([ATTN, 512, "MfmaFlopsBF16", 0.56e9])
    rows.append([SCAN, 1024, "MfmaUtil", 3.0])
    rows.append([SCAN, 1024, "MfmaFlopsBF16", 2.2e9])
    rows.append([COMBINE, 64, "MfmaUtil", 0.0])
    rows.append([COMBINE, 64, "MfmaFlopsBF16", 0.0])
    _write(os.path.join(mf, "run_counter_collection.csv"), ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"],
           rows)
    out = str(tmp_path / "out")
    os.makedirs(out)
    assert P.main(["--workload", "w", "--stats", st, "--mfma", mf, "--out-dir", out]) == 0
    md = open(os.path.join(out, "mfma_util_w.md")).read()
    # 0.56 GFLOP in 7 us = 80 TFLOP/s = 3.2 % of the bf16 peak; kernels without MFMA work are left out
    assert "| `herald::attn_kernel<128>` | 2 | 11.0 | 0.560 | 7.00 | 80.0 | 3.2 |" in md
    assert "| `herald::scan_mfma_kernel<128>` | 1 | 3.0 | 2.200 | 17.00 | 129.4 | 5.1 |" in md
    assert "attn_combine" not in md
