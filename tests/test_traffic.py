"""The counter reduction behind roofline.traffic (bf16_fp8_weight_amd.traffic)
on synthetic rocprofv3 CSVs: per-dispatch sums, calibration scales from a
copy of known size, and the kernel-source hash it is keyed by. CPU only."""
import csv
import json
import os
import subprocess
import sys

from bf16_fp8_weight_amd import traffic as T

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _csv(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "pmc_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(FIELDS, r)))


def test_readings_sum_per_dispatch_and_filter(tmp_path):
    d = str(tmp_path / "r")
    # two rows per dispatch (e.g. per-XCD instances) are summed; other kernels are ignored
    _csv(d, [(1, "wt::prep_fast_copy_kernel(x)", "FETCH_SIZE", 10.0), (1, "wt::prep_fast_copy_kernel(x)", "FETCH_SIZE", 5.0),
             (2, "other_kernel", "FETCH_SIZE", 99.0), (3, "wt::prep_fast_copy_kernel(x)", "FETCH_SIZE", 16.0),
             (3, "wt::prep_fast_copy_kernel(x)", "WRITE_SIZE", 7.0)])
    assert T.readings(d, "prep_fast_copy", "FETCH_SIZE") == [15.0, 16.0]
    assert T.readings(d, "prep_fast_copy", "WRITE_SIZE") == [7.0]


def test_scaled_traffic_and_hash(tmp_path):
    kib = 1024
    copy_bytes = 1000 * kib
    dirs = {k: str(tmp_path / k) for k in ("f", "w", "cf", "cw")}
    # the copy reads copy_bytes but FETCH_SIZE reports half; WRITE_SIZE is exact
    _csv(dirs["cf"], [(i, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 500.0) for i in range(3)])
    _csv(dirs["cw"], [(i, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1000.0) for i in range(3)])
    _csv(dirs["f"], [(i, "wt::prep_fast_copy_kernel", "FETCH_SIZE", 300.0) for i in range(3)])
    _csv(dirs["w"], [(i, "wt::prep_fast_copy_kernel", "WRITE_SIZE", 150.0) for i in range(3)])
    out = str(tmp_path / "traffic.json")
    subprocess.run([sys.executable, "-m", "bf16_fp8_weight_amd.traffic", "--kernel", "prep_fast_copy_kernel",
                    "--workload", "w", "--copy-bytes", str(copy_bytes), "--fetch", dirs["f"], "--write", dirs["w"],
                    "--copy-fetch", dirs["cf"], "--copy-write", dirs["cw"], "--out", out],
                   check=True, cwd=ROOT, capture_output=True)
    t = json.load(open(out))
    assert t["fetch_scale"] == 2.0 and t["write_scale"] == 1.0
    assert t["read_bytes"] == 600 * kib and t["write_bytes"] == 150 * kib and t["bytes_per_launch"] == 750 * kib
    assert t["kernel_source_sha"] == T.kernel_sha() and len(t["kernel_source_sha"]) == 16


def test_committed_traffic_matches_current_kernel_sources():
    # profiles/traffic.json must be re-measured whenever the kernel sources change
    t = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    assert t["kernel_source_sha"] == T.kernel_sha(), "kernel sources changed since the counters were taken"
    assert t["workload"] == "kimi_k2_moe_96experts"
    assert 1.0 <= t["bytes_per_launch"] / 12684607488 < 1.01
