"""Readers for the text fixtures under tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def e4m3_values():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3fn_values.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            rows.append((float(tok[0]), int(tok[1], 16)))
    return rows


def worked_tiles():
    tiles, cur = [], None
    with open(os.path.join(GOLDEN, "worked_tiles.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] == "tile":
                cur = {"name": tok[1], "rows": int(tok[2]), "cols": int(tok[3])}
                tiles.append(cur)
            elif tok[0] == "x":
                cur["x"] = np.array([float(t) for t in tok[1:]], dtype=np.float32).reshape(cur["rows"], cur["cols"])
            elif tok[0] == "scale_bits":
                cur["scale_bits"] = int(tok[1], 16)
            elif tok[0] == "bytes":
                cur["bytes"] = np.array([int(t, 16) for t in tok[1:]], dtype=np.uint8).reshape(cur["rows"], cur["cols"])
    return tiles


def f32_to_bf16_bits_exact(x):
    """BF16 bit patterns of float32 values that are exactly representable in BF16."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in BF16"
    return (u >> 16).astype(np.uint16)


def schedule_example():
    """tests/golden/schedule_example.txt as (params, dsts, expect, region, shards, unused);
    expect maps a tensor to (dst_offset, scale_offset, source, input_bytes)."""
    params, dsts, expect, shards = [], [], {}, {}
    region = unused = None
    with open(os.path.join(GOLDEN, "schedule_example.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] == "param":
                params.append({"name": tok[1], "rows": int(tok[2]), "cols": int(tok[3]), "n_shards": int(tok[4])})
            elif tok[0] == "dst":
                dsts.append({"name": tok[1], "dtype": 0 if tok[2] == "fp8" else 1, "components": tok[3:]})
            elif tok[0] == "expect":
                expect[tok[1]] = tuple(int(t) for t in tok[2:5])
            elif tok[0] == "inbytes":
                expect[tok[1]] = expect[tok[1]] + (int(tok[2]),)
            elif tok[0] == "region":
                region = int(tok[1])
            elif tok[0] == "shards":
                shards[tok[1]] = [int(t) for t in tok[2:]]
            elif tok[0] == "unused":
                unused = int(tok[1])
    return params, dsts, expect, region, shards, unused


def act_blocks():
    """tests/golden/act_blocks.txt as a list of dicts {name, cols, x, bytes, scale_bits}."""
    rows, cur = [], None
    with open(os.path.join(GOLDEN, "act_blocks.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] == "row":
                cur = {"name": tok[1], "cols": int(tok[2])}
                rows.append(cur)
            elif tok[0] == "x":
                x = np.zeros(cur["cols"], dtype=np.uint16)
                for t in tok[1:]:
                    c, v = t.split(":")
                    x[int(c)] = int(v, 16)
                cur["x"] = x
            elif tok[0] == "bytes":
                cur["bytes"] = {int(c): int(v, 16) for c, v in (t.split(":") for t in tok[1:])}
            elif tok[0] == "scale_bits":
                cur["scale_bits"] = [int(t, 16) for t in tok[1:]]
    return rows
