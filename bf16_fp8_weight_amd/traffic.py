"""HBM traffic of a kernel from rocprofv3 counter runs, for the roofline line.

Four runs, one counter each (rocprofv3 --pmc <C> --output-format csv): the
kernel with FETCH_SIZE, then WRITE_SIZE, and a plain device copy of a known
byte count (bench.py --calibrate-copy BYTES) with each counter. A counter's
scale is the copy's known bytes over what the counter reports for it; the
kernel's traffic per launch is its per-dispatch readings (KiB) times those
scales. The result goes to profiles/traffic.json with the hash of the kernel
sources it was measured with (their code, comments and layout left out);
bench.py reports it only while the hash still matches.

    python -m bf16_fp8_weight_amd.traffic --kernel prep_fast_copy_kernel \\
        --workload kimi_k2_moe_96experts --copy-bytes 4228890624 \\
        --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR [--out profiles/traffic.json]
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
# sources whose change invalidates a traffic measurement of the preparation kernel
KERNEL_SOURCES = ("prep_kernels.hip", "fp8_math.h", "wt_internal.h")


def _code_only(text: str) -> str:
    """Source text without comments and with whitespace collapsed, so that a
    comment edit does not invalidate a measurement of unchanged code."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(PKG, "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def readings(run_dir: str, kernel_substr: str, counter: str) -> list:
    """Per-dispatch values (KiB) of `counter` for kernels whose name contains kernel_substr."""
    path = os.path.join(run_dir, "pmc_counter_collection.csv")
    by_dispatch = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if kernel_substr in row["Kernel_Name"] and row["Counter_Name"] == counter:
                d = row["Dispatch_Id"]
                by_dispatch[d] = by_dispatch.get(d, 0.0) + float(row["Counter_Value"])
    if not by_dispatch:
        raise SystemExit(f"no {counter} readings for '{kernel_substr}' in {path}")
    return [by_dispatch[k] for k in sorted(by_dispatch, key=int)]


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--kernel", required=True, help="substring of the kernel's name")
    ap.add_argument("--workload", required=True, help="workload name as bench.py reports it")
    ap.add_argument("--copy-bytes", type=int, required=True)
    ap.add_argument("--copy-kernel", default="copyBuffer")
    for k in ("fetch", "write", "copy-fetch", "copy-write"):
        ap.add_argument("--" + k, required=True, metavar="DIR")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles", "traffic.json"))
    a = ap.parse_args()

    kib = a.copy_bytes / 1024.0
    fetch_scale = kib / statistics.median(readings(a.copy_fetch, a.copy_kernel, "FETCH_SIZE"))
    write_scale = kib / statistics.median(readings(a.copy_write, a.copy_kernel, "WRITE_SIZE"))
    f = readings(a.fetch, a.kernel, "FETCH_SIZE")
    w = readings(a.write, a.kernel, "WRITE_SIZE")
    fk, wk = statistics.median(f), statistics.median(w)
    rd, wr = fk * 1024 * fetch_scale, wk * 1024 * write_scale
    out = {
        "workload": a.workload, "kernel": a.kernel, "kernel_source_sha": kernel_sha(),
        "bytes_per_launch": int(round(rd + wr)), "read_bytes": int(round(rd)), "write_bytes": int(round(wr)),
        "fetch_size_kib": fk, "write_size_kib": wk, "fetch_scale": fetch_scale, "write_scale": write_scale,
        "fetch_size_kib_per_dispatch": f, "write_size_kib_per_dispatch": w,
    }
    with open(a.out, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
