"""Turns a workload (bf16_fp8_weight_amd.workloads) into the oracle's input.

Test-side glue only: it copies each shard's bytes to host numpy arrays and
hands them to ``oracle.prepare``. It performs none of the preparation.
"""
import numpy as np
import torch

import oracle
from bf16_fp8_weight_amd import workloads as W


def shard_bits(t: torch.Tensor) -> np.ndarray:
    a = t.detach()
    if a.device.type != "cpu":
        a = a.cpu()
    a = a.contiguous().view(torch.int16).numpy().view(np.uint16)
    if a.ndim == 1:
        a = a.reshape(-1, 1)
    return a


def oracle_outputs(wl: W.Workload):
    outs = []
    for o in wl.outputs:
        parts = [[shard_bits(s).reshape(-1, o.cols) for s in p.shards] for p in o.parts]
        kind = oracle.FP8_TILE128 if o.kind == W.FP8 else oracle.BF16_COPY
        outs.append(oracle.Output(kind, o.cols, parts, o.dst_offset, o.scale_offset))
    return outs


def oracle_image(wl: W.Workload, fill: int = 0) -> np.ndarray:
    dst = np.full(wl.dst_bytes, fill, dtype=np.uint8)
    return oracle.prepare(oracle_outputs(wl), wl.dst_bytes, dst)


def full_bits(part: W.Part, cols: int) -> np.ndarray:
    """The assembled component as host bits, via torch.cat of its shards."""
    return shard_bits(torch.cat([s.reshape(-1, cols).cpu() for s in part.shards], dim=0)).reshape(-1, cols)
