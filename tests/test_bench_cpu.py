"""The benchmark's host-side contract, without a GPU: the one-GPU rule, the
CPU-baseline timing helper and the source hash that gates the committed HBM
traffic record."""
import json
import os
import subprocess
import sys

import bench
from fp32_gemm_major_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and "--gpus must be 1" in p.stderr
    assert p.stdout == ""


def test_time_oracle_on_a_small_problem():
    ops = wl.operands(wl.Workload("t", 7, 64, 48, 40, 1.0, 0.0, "uniform"))
    gflops, rows, reps, seconds = bench.time_oracle(ops, 0.05, 1)
    assert gflops > 0 and 1 <= rows <= 64 and reps >= 1 and seconds > 0


def test_time_oracle_repeats_a_short_whole_problem():
    """A problem whose whole run is far under the target is repeated, so the
    figure does not rest on a single run of a few milliseconds."""
    ops = wl.operands(wl.Workload("t", 9, 32, 32, 32, 1.0, 0.0, "uniform"))
    gflops, rows, reps, seconds = bench.time_oracle(ops, 0.2, 1)
    assert rows == 32 and reps >= 2 and seconds >= 0.1 and gflops > 0


def test_cpu_baseline_fields():
    ops = wl.operands(wl.Workload("t", 8, 96, 64, 32, 1.5, 0.5, "uniform"))
    cb = bench.cpu_baseline(ops, 0.05)
    assert cb["kind"] == "oracle" and cb["unit"] == "GFLOPS" and cb["value"] > 0
    assert cb["cores"] >= 1 and "rows 0.." in cb["sample"]
    assert set(cb["single_core"]) == {"c1_128", "c2_1024", "c4_edge"}
    for v in cb["single_core"].values():
        assert v["gflops"] > 0 and 1 <= v["rows"] <= v["of_rows"] and v["repetitions"] >= 1


def test_kernel_source_hash_and_traffic_record():
    hm = bench.kernel_source_hash("mfma_M256x128_aligned")
    hv = bench.kernel_source_hash("valu_V128x128_aligned")
    assert len(hm) == 16 and hm != hv
    assert hm == bench.kernel_source_hash("mfma_M64x64_edge")  # one family, one hash
    with open(os.path.join(ROOT, "profiles", "traffic.json"), encoding="utf-8") as f:
        entries = json.load(f)["entries"]
    for e in entries:
        assert e["fetch_scale"] > 0 and e["write_scale"] > 0
        # the stored counts and scales are rounded; the total is not
        total = (e["fetch_kib_raw"] * e["fetch_scale"]
                 + e["write_kib_raw"] * e["write_scale"]) * 1024
        assert abs(e["hbm_bytes_per_launch"] - total) <= 1e-4 * total
