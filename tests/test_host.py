"""Host-side logic without a GPU: the bench's one-GPU contract, the seeded
input generators, and the rocprofv3 summary arithmetic."""
import csv
import os
import subprocess
import sys

import numpy as np

from collective_reduction_ring_amd import profiling
from collective_reduction_ring_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


def test_generators_are_seeded_and_thread_independent():
    a = wl.rank_inputs(1)
    b = [wl.draw("uniform", wl.rng_for(1, r), 4096) for r in range(4)]
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    g1, a1 = wl.sparse_inputs(n=1000, world=3)
    g2, a2 = wl.sparse_inputs(n=1000, world=3)
    assert all(np.array_equal(x, y) for x, y in zip(g1 + a1, g2 + a2))
    assert not np.array_equal(g1[0], a1[0])
    assert g1[0].dtype == np.float32 and abs(float(np.std(g1[0])) - 1e-3) < 1e-4


def test_fused_sizes_log_uniform_in_range():
    s = wl.fused_sizes()
    assert len(s) == wl.FUSED_COUNT and s.min() >= wl.FUSED_MIN and s.max() <= wl.FUSED_MAX
    assert np.array_equal(s, wl.fused_sizes())
    # log-uniform: about half the sizes below the geometric mean of the bounds
    assert 0.35 < np.mean(s < np.sqrt(wl.FUSED_MIN * wl.FUSED_MAX)) < 0.65


def test_bf16_bucket_size():
    assert wl.BF16_BUCKET_ELEMS * 2 == 25 * 2 ** 20
    assert wl.WORKLOADS[3].n % wl.BF16_BUCKET_ELEMS == 3_145_728


def _write(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_ktrace_summary_timed_window(tmp_path):
    trace = tmp_path / "t.csv"
    stats = tmp_path / "s.csv"
    rows = []
    for i in range(6):  # durations 10, 11, ..., 15 us of the kernel, plus another kernel
        rows.append({"Kernel_Name": "fold_kernel<x>", "Start_Timestamp": 1000 * i * 100,
                     "End_Timestamp": 1000 * i * 100 + 1000 * (10 + i)})
        rows.append({"Kernel_Name": "other", "Start_Timestamp": 1000 * i * 100 + 50,
                     "End_Timestamp": 1000 * i * 100 + 60})
    _write(trace, rows)
    _write(stats, [{"Name": "fold_kernel<x>", "Calls": 6, "AverageNs": 12500, "MinNs": 10000,
                    "MaxNs": 15000, "Percentage": 99.0}])
    text = profiling.ktrace_summary(str(trace), str(stats), "fold_kernel", 2, 3, "cmd")
    # dispatches 2..4 of the kernel: 12, 13, 14 us
    assert "**13.0 us**" in text and "dispatches 2..4" in text and "cmd" in text


def test_traffic_record_scales_by_the_copy_calibration(tmp_path):
    def counters(path, name, kernel, kib):
        _write(path, [{"Counter_Name": name, "Kernel_Name": kernel, "Counter_Value": v} for v in kib])
    counters(tmp_path / "f.csv", "FETCH_SIZE", "fold", [500.0, 500.0])
    counters(tmp_path / "w.csv", "WRITE_SIZE", "fold", [250.0])
    counters(tmp_path / "cf.csv", "FETCH_SIZE", "copy", [512.0])     # a 1 MiB copy reads 1 MiB: scale 2
    counters(tmp_path / "cw.csv", "WRITE_SIZE", "copy", [1024.0])    # and writes 1 MiB: scale 1
    rec = profiling.traffic_record(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                                   str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"),
                                   "fold", "copy", 1 << 20, 1_280_000, "cmds")
    assert rec["fetch_bytes_per_launch"] == 1_024_000
    assert rec["write_bytes_per_launch"] == 256_000
    assert rec["traffic_over_algorithmic"] == 1.0
    assert rec["kernel_source_sha256"] == profiling.kernel_source_digest()


def test_traffic_table_scales_each_kernel(tmp_path):
    def counters(path, name, rows):
        _write(path, [{"Counter_Name": name, "Kernel_Name": k, "Counter_Value": v} for k, v in rows])
    counters(tmp_path / "f.csv", "FETCH_SIZE", [("gather<1>", 100.0), ("gather<1>", 300.0), ("combine", 10.0)])
    counters(tmp_path / "w.csv", "WRITE_SIZE", [("gather<1>", 50.0), ("combine", 40.0)])
    counters(tmp_path / "cf.csv", "FETCH_SIZE", [("copy", 512.0)])    # scale 2
    counters(tmp_path / "cw.csv", "WRITE_SIZE", [("copy", 1024.0)])   # scale 1
    text = profiling.traffic_table(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "cf.csv"),
                                   str(tmp_path / "cw.csv"), "copy", 1 << 20,
                                   [("gather", 460_800), ("combine", 61_440)], "cmds")
    # gather: fetch mean 200 KiB x 2 = 409,600 B, write 51,200 B -> 460,800 = 1.0000
    assert "| `gather` | 2 | 409,600 | 51,200 | 460,800 | 460,800 | 1.0000 |" in text
    # combine: 10 KiB x 2 + 40 KiB = 20,480 + 40,960 = 61,440
    assert "| `combine` | 1 | 20,480 | 40,960 | 61,440 | 61,440 | 1.0000 |" in text
