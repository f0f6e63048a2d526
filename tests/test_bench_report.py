"""Host logic of bench_report.py (the profile summaries): the copy
calibration of the traffic counters, the per-kernel sums and the derived
counter shares, on small synthetic rocprofv3-style CSV files."""
import csv
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def _counter_rows(counter, per_kernel):
    rows, d = [], 0
    for name, grid, values in per_kernel:
        for v in values:
            d += 1
            # two partial records per dispatch (as for per-XCD counters)
            for part in (v / 2, v / 2):
                rows.append({"Dispatch_Id": d, "Kernel_Name": name, "Grid_Size": grid, "Counter_Name": counter,
                             "Counter_Value": part})
    return rows


def _run(args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench_report.py"), *args], capture_output=True,
                       text=True)
    assert r.returncode == 0, r.stderr
    return r.stdout


def test_traffic_calibration_and_totals(tmp_path):
    gib_kib = 1 << 20
    # the copy reads FETCH_SIZE at half its size and WRITE_SIZE at full size
    fetch = _counter_rows("FETCH_SIZE", [("__amd_rocclr_copyBuffer", 131072, [gib_kib / 2] * 3),
                                         ("void k_t<1>(Args)", 4096, [1000.0, 1000.0])])
    write = _counter_rows("WRITE_SIZE", [("__amd_rocclr_copyBuffer", 131072, [gib_kib] * 3),
                                         ("void k_t<1>(Args)", 4096, [500.0, 500.0])])
    _write(tmp_path / "f.csv", fetch)
    _write(tmp_path / "w.csv", write)
    out = _run(["traffic", "--fetch", str(tmp_path / "f.csv"), "--write", str(tmp_path / "w.csv"),
                "--kernel", "k_t<", "--algorithmic", "3072000", "--workload", "w", "--source-sha", "abc"])
    kv = dict(line.split(": ", 1) for line in out.splitlines() if ": " in line and not line.startswith("#"))
    assert kv["fetch_scale"] == "2.0000" and kv["write_scale"] == "1.0000"
    # 1000 KiB x 2 read + 500 KiB x 1 written = 2500 KiB = 2,560,000 bytes
    assert int(kv["hbm_bytes_per_launch"]) == 2_560_000
    assert kv["kernel_source_sha"] == "abc"


def test_counter_shares(tmp_path):
    rows = []
    for c, v in (("GRBM_GUI_ACTIVE", 8000.0), ("TA_TA_BUSY_sum", 256000.0 / 2), ("TCC_HIT_sum", 30.0),
                 ("TCC_MISS_sum", 10.0), ("SQ_LDS_BANK_CONFLICT", 10.0), ("SQ_LDS_IDX_ACTIVE", 50.0),
                 ("SQ_VALU_MFMA_BUSY_CYCLES", 1024000.0 / 4)):
        rows.append({"Dispatch_Id": 1, "Kernel_Name": "void k_t<1>(Args)", "Grid_Size": 64, "Counter_Name": c,
                     "Counter_Value": v})
    _write(tmp_path / "c.csv", rows)
    out = _run(["counters", str(tmp_path / "c.csv"), "--kernel", "k_t<"])
    assert "TA busy share per CU: 50.0 %" in out          # 128000 / 256 / (8000 / 8)
    assert "L2 hit rate: 75.0 %" in out
    assert "LDS bank conflict ratio (conflict cycles / conflict-free active cycles): 0.250" in out
    assert "MFMA busy share per SIMD: 25.00 %" in out     # 256000 / (1000 * 1024)
