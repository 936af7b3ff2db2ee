"""Helpers for the GPU tests: run the library on a workload, run the oracle
on the same bytes (threaded over outputs), compare images."""
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
import oracle_glue

WORKERS = min(16, os.cpu_count() or 1)


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_library(wl, fill=0xA5, dst_kind=None, opts=None, table=None, stream=None):
    from bf16_fp8_weight_amd import wt

    kind = wt.WT_MEM_DEVICE if dst_kind is None else dst_kind
    if kind == wt.WT_MEM_DEVICE:
        dst = torch.full((wl.dst_bytes,), fill, dtype=torch.uint8, device="cuda")
    else:
        dst = torch.full((wl.dst_bytes,), fill, dtype=torch.uint8).pin_memory()
    tab = table if table is not None else wt.task_table(wl)
    h = wt.wt_plan_create(tab, dst.data_ptr(), wl.dst_bytes, kind, opts)
    try:
        s = stream if stream is not None else torch.cuda.current_stream()
        wt.wt_prepare(h, s.cuda_stream)
        s.synchronize()
        info = wt.wt_plan_get_info(h)
    finally:
        wt.wt_plan_destroy(h)
    return dst.cpu().numpy(), info


def oracle_image_threaded(wl, fill=0xA5, outputs=None):
    outs = oracle_glue.oracle_outputs(wl)
    if outputs is not None:
        outs = [outs[i] for i in outputs]
    img = np.full(wl.dst_bytes, fill, dtype=np.uint8)
    with ThreadPoolExecutor(WORKERS) as ex:
        list(ex.map(lambda o: oracle.prepare([o], wl.dst_bytes, img), outs))
    return img


def assert_images_equal(got, want, wl):
    if np.array_equal(got, want):
        return
    bad = np.nonzero(got != want)[0]
    where = []
    for b in bad[:5]:
        for o in wl.outputs:
            if o.dst_offset <= b < o.dst_offset + o.data_bytes:
                e = b - o.dst_offset
                r, c = (e // o.cols, e % o.cols) if o.kind == "fp8" else (e // (2 * o.cols), (e // 2) % o.cols)
                where.append(f"{o.name} data r{r} c{c}: got {got[b]:#04x} want {want[b]:#04x}")
                break
            if o.kind == "fp8" and o.scale_offset <= b < o.scale_offset + o.scale_bytes:
                t = (b - o.scale_offset) // 4
                where.append(f"{o.name} scale tile {t}")
                break
        else:
            where.append(f"byte {b} outside every range: got {got[b]:#04x} want {want[b]:#04x}")
    raise AssertionError(f"{bad.size} bytes differ; first: " + "; ".join(where))


class Timer:
    def __init__(self, what):
        self.what = what

    def __enter__(self):
        self.t = time.time()
        return self

    def __exit__(self, *a):
        log(f"  [{self.what}: {time.time() - self.t:.1f}s]")
