"""Host logic of bench.py on small synthetic profiler outputs (CPU only): the per-kernel counter
reduction (MFMA utilisation, clock, copy-scaled HBM bytes) and the sparse pair count."""
import csv
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

COUNTER_COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
                "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size",
                "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value",
                "Start_Timestamp", "End_Timestamp"]
TRACE_COLS = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id",
              "Kernel_Name", "Correlation_Id", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size",
              "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Workgroup_Size_X",
              "Workgroup_Size_Y", "Workgroup_Size_Z", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
ATT = "void qvd::k_sparse_attn<1>(args)"
COPY = "__amd_rocclr_copyBuffer"


def _write(path, cols, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow({c: r.get(c, 0) for c in cols})


def _counter_rows(per_dispatch):
    """per_dispatch: [(dispatch id, kernel, grid, {counter: [values per XCD/instance]})]"""
    rows = []
    for did, name, grid, counters in per_dispatch:
        for cname, vals in counters.items():
            for v in vals:
                rows.append({"Dispatch_Id": did, "Kernel_Name": name, "Grid_Size": grid,
                             "Counter_Name": cname, "Counter_Value": v})
    return rows


def test_parse_counters_table(tmp_path, capsys):
    grid = 2772 * 512
    # two attention dispatches: GRBM summed over 8 XCDs (8 x 1e6 cycles), MFMA busy 1024 SIMDs x 5e5
    mfma = [(10 + i, ATT, grid, {"GRBM_GUI_ACTIVE": [1e6] * 8, "SQ_VALU_MFMA_BUSY_CYCLES": [1024 * 5e5]})
            for i in range(2)]
    _write(str(tmp_path / "m" / "p_counter_collection.csv"), COUNTER_COLS, _counter_rows(mfma))
    # the 1 GiB probe copy reads as 512 Ki KiB fetched (factor 2) and 1 Mi KiB written (factor 1)
    fetch = [(10, ATT, grid, {"FETCH_SIZE": [250_000.0, 250_000.0]}), (11, ATT, grid, {"FETCH_SIZE": [500_000.0]}),
             (20, COPY, 1 << 16, {"FETCH_SIZE": [524_288.0]})]
    write = [(10, ATT, grid, {"WRITE_SIZE": [100_000.0]}), (11, ATT, grid, {"WRITE_SIZE": [100_000.0]}),
             (20, COPY, 1 << 16, {"WRITE_SIZE": [1_048_576.0]})]
    _write(str(tmp_path / "f" / "p_counter_collection.csv"), COUNTER_COLS, _counter_rows(fetch))
    _write(str(tmp_path / "w" / "p_counter_collection.csv"), COUNTER_COLS, _counter_rows(write))
    # trace: the step starts at the AdaLN projection; two attention launches of 500 us (1e6 cycles at
    # 2 GHz), then a 768p-like attention launch of another grid that must not be counted
    tr = [{"Dispatch_Id": 1, "Kernel_Name": "qvd::k_adaln_project(args)", "Start_Timestamp": 0,
           "End_Timestamp": 1000, "Grid_Size_X": 63 * 256, "Grid_Size_Y": 42, "Grid_Size_Z": 1}]
    for i in range(2):
        t0 = 10_000 + i * 1_000_000
        tr.append({"Dispatch_Id": 2 + i, "Kernel_Name": ATT, "Start_Timestamp": t0, "End_Timestamp": t0 + 500_000,
                   "Grid_Size_X": grid, "Grid_Size_Y": 1, "Grid_Size_Z": 1})
    tr.append({"Dispatch_Id": 99, "Kernel_Name": ATT, "Start_Timestamp": 9_000_000_000, "End_Timestamp": 9_009_000_000,
               "Grid_Size_X": 7 * 512, "Grid_Size_Y": 1, "Grid_Size_Z": 1})
    _write(str(tmp_path / "t" / "run_kernel_trace.csv"), TRACE_COLS, tr)

    bench.parse_counters(str(tmp_path / "m"), str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "t"))
    out = capsys.readouterr().out
    row = [l for l in out.splitlines() if "k_sparse_attn<1>" in l]
    assert len(row) == 1, out
    cells = [c.strip() for c in row[0].split("|")[1:-1]]
    # dispatches, cycles (8e6 / 8 XCDs), us, clock, busy = 5e5 / 1e6, busy x clock / 2.4
    assert cells[2] == "2" and cells[3] == "1,000,000" and cells[4] == "500.0" and cells[5] == "2.00"
    assert cells[6] == "50.0%" and cells[7] == f"{100 * 0.5 * 2.0 / 2.4:.1f}%"
    # bytes: mean fetch 500,000 KiB x 1024 x 2 + write 100,000 KiB x 1024 x 1
    gb = (500_000 * 1024 * 2 + 100_000 * 1024) / 1e9
    assert cells[8] == f"{gb:.3f}" and cells[9] == f"{gb / 500.0 * 1e3:.2f}"


def test_kept_scores_counts_ragged_tiles():
    # 300 tokens: tiles of 128, 128, 44 rows; one head keeping tiles {0, 2} for every query tile
    L = 300
    idx = np.array([[[0, 2], [0, 2], [0, 2]]], np.int32)
    cnt = np.array([[2, 2, 2]], np.int32)
    rows = [128, 128, 44]
    want = sum(rq * (rows[0] + rows[2]) for rq in rows)
    assert bench.kept_scores(idx, cnt, L) == want
