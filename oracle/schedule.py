"""Plain reference of the static transfer schedule (test infrastructure only).

What the controller computes ("Weight transfer for RL post-training in under
2 seconds", section "High-level workflow": metadata from training and
inference, then a static schedule of which training GPU sends which
parameter where; section "Static schedule"). Readings of what the page leaves
open, taken identically by the library:
  - a fused inference tensor is the dim-0 concatenation of its training
    parameters in the listed order; all share cols;
  - FSDP shards are the torch.chunk split of the rows: ceil(rows / n) rows
    each, trailing shards smaller or empty, always n shards;
  - destination layout: inference tensors in their listed order, each one's
    data then (FP8 only) its fp32 scale grid of ceil(R/128) x ceil(C/128),
    every range starting at the next multiple of `align`; region size rounded
    up to `align`;
  - source GPUs: longest processing time first over BF16 input bytes (ties
    keep the listed order), each output to the least-loaded source (ties to
    the lowest index).
Nothing here is shared with the library.
"""
from __future__ import annotations

FP8 = 0
BF16 = 1


def chunk_rows(rows: int, n: int) -> list:
    per = -(-rows // n)
    out, left = [], rows
    for _ in range(n):
        r = min(per, left)
        out.append(r)
        left -= r
    return out


def build(params: list, dsts: list, align: int = 256, n_sources: int = 1) -> dict:
    """params: [{name, rows, cols, n_shards}], dsts: [{name, components, dtype}].
    Returns {outputs: [{dst_offset, scale_offset, source, input_bytes, rows,
    cols, components}], dst_bytes, tasks: [{param, shard_rows, cols, dtype,
    fusion_group, dst_offset, scale_offset, output}], n_unused}."""
    by_name = {p["name"]: p for p in params}
    if len(by_name) != len(params):
        raise ValueError("duplicate parameter name")
    used = set()
    outputs, cursor = [], 0

    def up(x):
        return -(-x // align) * align

    for d in dsts:
        comps = [by_name[c] for c in d["components"]]
        cols = comps[0]["cols"]
        if any(c["cols"] != cols for c in comps):
            raise ValueError("fusion components differ in cols")
        rows = sum(c["rows"] for c in comps)
        used.update(d["components"])
        o = {"rows": rows, "cols": cols, "components": list(d["components"]), "dtype": d["dtype"],
             "input_bytes": 2 * rows * cols}
        cursor = up(cursor)
        o["dst_offset"] = cursor
        cursor += rows * cols * (1 if d["dtype"] == FP8 else 2)
        o["scale_offset"] = 0
        if d["dtype"] == FP8:
            cursor = up(cursor)
            o["scale_offset"] = cursor
            cursor += 4 * (-(-rows // 128)) * (-(-cols // 128))
        outputs.append(o)
    dst_bytes = up(cursor)

    load = [0] * n_sources
    order = sorted(range(len(outputs)), key=lambda i: -outputs[i]["input_bytes"])  # stable: ties keep order
    for i in order:
        s = min(range(n_sources), key=lambda k: (load[k], k))
        outputs[i]["source"] = s
        load[s] += outputs[i]["input_bytes"]

    tasks = []
    for oi, (d, o) in enumerate(zip(dsts, outputs)):
        for c in d["components"]:
            p = by_name[c]
            tasks.append({"param": c, "shard_rows": chunk_rows(p["rows"], p["n_shards"]), "cols": p["cols"],
                          "dtype": d["dtype"], "fusion_group": oi if len(d["components"]) > 1 else -1,
                          "dst_offset": o["dst_offset"], "scale_offset": o["scale_offset"], "output": oi})
    return {"outputs": outputs, "dst_bytes": dst_bytes, "tasks": tasks,
            "n_unused": sum(1 for p in params if p["name"] not in used)}
