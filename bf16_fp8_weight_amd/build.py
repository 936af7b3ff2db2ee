"""Builds libwt.so (host plan + runtime + gfx950 kernels) in-tree with hipcc.

Flags: -O3 for gfx950 only; no fast-math and no denormal flushing (subnormal
scales and inputs are part of the contract); packed-fp32 instruction
selection disabled for device code.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libwt.so")

SOURCES = ["plan.cpp", "schedule.cpp", "host_api.cpp", "runtime.cpp", "prep_kernels.hip", "progress.hip", "act_quant.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-std=c++17", "-O3", "-fPIC", "-Wall", "-Wno-unused-function",
    "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-I", INCLUDE, "-I", CSRC,
]
DEVICE = ["-x", "hip", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False, save_temps_dir: str | None = None, defines=(), out: str | None = None) -> str:
    """Compiles every source and links libwt.so (or `out`). Always rebuilds.
    `defines` are extra -D options (kernel tuning knobs)."""
    objdir = os.path.join(ROOT, "_build", "default" if not defines else "_".join(d.replace("=", "") for d in defines))
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(objdir, src + ".o")
        cmd = [HIPCC, *COMMON, *DEVICE, *("-D" + d for d in defines), "-c", path, "-o", obj]
        if save_temps_dir and src.endswith(".hip"):
            cmd += ["-save-temps=obj"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, cwd=save_temps_dir or objdir)
        objs.append(obj)
    target = out or LIB_PATH
    tmp = target + ".tmp%d" % os.getpid()
    link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, target)
    return target


if __name__ == "__main__":
    import argparse

    ap = argparse.ArgumentParser()
    ap.add_argument("-v", action="store_true")
    ap.add_argument("-D", action="append", default=[], help="extra define, e.g. -D WT_SAT_CLAMP=0")
    ap.add_argument("-o", default=None, help="output library path")
    a = ap.parse_args()
    print(build(verbose=a.v, defines=a.D, out=a.o))
