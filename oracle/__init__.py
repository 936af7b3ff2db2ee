"""Python access to the CPU oracle (``oracle.c``) for parameter preparation.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does. It
marshals numpy arrays into the C structs of ``oracle.h`` and nothing else; it
imports nothing from the GPU library.

The definition it computes ("Weight transfer for RL post-training in under 2
seconds", section "Task pipeline": rebuild the full weight, fuse projections,
quantize) and the readings of what the page leaves open are in ``oracle.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field
from typing import List, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# WT_ORACLE_LIB lets the mutation test load a deliberately broken copy of the
# oracle (built from a patched copy of oracle.c in a temporary directory).
LIB_PATH = os.environ.get("WT_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")

FP8_TILE128 = 0
BF16_COPY = 1

_CFLAGS = ["-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no flush-to-zero flags)."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", *_CFLAGS, os.path.join(HERE, "oracle.c"), "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


class _Shard(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("rows", ctypes.c_int64)]


class _Part(ctypes.Structure):
    _fields_ = [("shards", ctypes.POINTER(_Shard)), ("n_shards", ctypes.c_int32)]


class _Output(ctypes.Structure):
    _fields_ = [
        ("parts", ctypes.POINTER(_Part)),
        ("n_parts", ctypes.c_int32),
        ("kind", ctypes.c_int32),
        ("cols", ctypes.c_int64),
        ("dst_offset", ctypes.c_uint64),
        ("scale_offset", ctypes.c_uint64),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_e4m3fn_from_f32.restype = ctypes.c_uint8
        L.oracle_e4m3fn_from_f32.argtypes = [ctypes.c_float]
        L.oracle_e4m3fn_value.restype = ctypes.c_double
        L.oracle_e4m3fn_value.argtypes = [ctypes.c_uint8]
        L.oracle_tile_scale.restype = ctypes.c_float
        L.oracle_tile_scale.argtypes = [ctypes.c_float]
        L.oracle_quantize_element.restype = ctypes.c_uint8
        L.oracle_quantize_element.argtypes = [ctypes.c_uint16, ctypes.c_float]
        L.oracle_prepare.restype = ctypes.c_int
        L.oracle_prepare.argtypes = [ctypes.POINTER(_Output), ctypes.c_int64, ctypes.c_void_p, ctypes.c_uint64]
        L.oracle_quantize_domain.restype = None
        L.oracle_quantize_domain.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        L.oracle_cast_f32_range.restype = None
        L.oracle_cast_f32_range.argtypes = [ctypes.c_uint32, ctypes.c_uint64, ctypes.c_void_p]
        L.oracle_cast_f32_array.restype = None
        L.oracle_cast_f32_array.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        L.oracle_quantize_elements.restype = None
        L.oracle_quantize_elements.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p]
        L.oracle_quantize_act_b128.restype = ctypes.c_int
        L.oracle_quantize_act_b128.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                               ctypes.c_void_p, ctypes.c_int64]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# ---------------------------------------------------------------- elementwise
def cast_e4m3fn(values) -> np.ndarray:
    """fp32 values -> E4M3 bytes (RNE, saturating), same shape."""
    v = np.ascontiguousarray(values, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().oracle_cast_f32_array(_ptr(v), v.size, _ptr(out))
    return out


def cast_f32_range(first: int, count: int) -> np.ndarray:
    """E4M3 bytes of the fp32 bit patterns first .. first+count-1."""
    out = np.empty(count, dtype=np.uint8)
    lib().oracle_cast_f32_range(first, count, _ptr(out))
    return out


def e4m3fn_value(byte: int) -> float:
    return lib().oracle_e4m3fn_value(byte)


def tile_scale(amax: float) -> float:
    return lib().oracle_tile_scale(amax)


def quantize_elements(x_bits, s: float) -> np.ndarray:
    """cast(fl32(x / s)) for BF16 bit patterns x and one fp32 scale s."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().oracle_quantize_elements(_ptr(x), x.size, float(s), _ptr(out))
    return out


def quantize_domain(amax_bits) -> np.ndarray:
    """[len(amax_bits), 65536] bytes: every BF16 x against the scale of each amax."""
    a = np.ascontiguousarray(amax_bits, dtype=np.uint16)
    out = np.empty((a.size, 65536), dtype=np.uint8)
    lib().oracle_quantize_domain(_ptr(a), a.size, _ptr(out))
    return out


# ------------------------------------------------------------------- prepare
@dataclass
class Output:
    """One output tensor for the oracle.

    parts: the fusion components in order; each is the list of its dim-0
    shards in rank order, every shard a uint16 array of BF16 bit patterns
    shaped (rows, cols) (a 1-D shard counts as (n, 1)).
    """

    kind: int
    cols: int
    parts: List[List[np.ndarray]]
    dst_offset: int
    scale_offset: int = 0
    _keep: list = field(default_factory=list, repr=False)


def prepare(outputs: Sequence[Output], dst_bytes: int, dst: np.ndarray | None = None) -> np.ndarray:
    """Runs oracle_prepare over `outputs` into a host image of dst_bytes bytes.

    `dst` (uint8, dst_bytes long) may be passed in pre-filled (for canary
    checks); otherwise a zero-filled image is returned.
    """
    if dst is None:
        dst = np.zeros(dst_bytes, dtype=np.uint8)
    assert dst.dtype == np.uint8 and dst.size == dst_bytes and dst.flags.c_contiguous
    keep = []
    outs = (_Output * max(1, len(outputs)))()
    for i, o in enumerate(outputs):
        parts = (_Part * len(o.parts))()
        for p, shards in enumerate(o.parts):
            arr = (_Shard * len(shards))()
            for k, sh in enumerate(shards):
                sh = np.ascontiguousarray(sh, dtype=np.uint16)
                keep.append(sh)
                rows = sh.shape[0] if sh.ndim >= 1 else 1
                if sh.ndim == 2:
                    assert sh.shape[1] == o.cols, "shard column count differs from the output's"
                arr[k].data = _ptr(sh) if sh.size else None
                arr[k].rows = rows
            keep.append(arr)
            parts[p].shards = ctypes.cast(arr, ctypes.POINTER(_Shard))
            parts[p].n_shards = len(shards)
        keep.append(parts)
        outs[i].parts = ctypes.cast(parts, ctypes.POINTER(_Part))
        outs[i].n_parts = len(o.parts)
        outs[i].kind = o.kind
        outs[i].cols = o.cols
        outs[i].dst_offset = o.dst_offset
        outs[i].scale_offset = o.scale_offset
    rc = lib().oracle_prepare(outs, len(outputs), _ptr(dst), dst_bytes)
    if rc != 0:
        raise ValueError("oracle_prepare failed with code %d" % rc)
    return dst


def quantize_act(x: np.ndarray, cols: int | None = None, index=None, n_out: int | None = None,
                 q: np.ndarray | None = None, scales: np.ndarray | None = None):
    """oracle_quantize_act_b128 on a host array.

    x: uint16 BF16 bits [n_rows, x_stride]; cols (default x_stride) columns
    used. index: int32 output-row -> input-row map, or None. q: uint8
    [n_out, q_stride] and scales: uint8 [n_out, s_stride] (pre-filled for
    canary checks) or None for zero-filled [n_out, cols] and
    [n_out, 4 ceil(cols / 128)]. Returns (q, scales as float32 view when
    s_stride is 4 ceil(cols / 128), else the raw bytes).
    """
    x = np.ascontiguousarray(x, dtype=np.uint16)
    assert x.ndim == 2
    n_rows, x_stride = x.shape
    cols = x_stride if cols is None else cols
    idx = None if index is None else np.ascontiguousarray(index, dtype=np.int32)
    n_out = (n_rows if idx is None else idx.size) if n_out is None else n_out
    nb = -(-cols // 128)
    if q is None:
        q = np.zeros((n_out, cols), dtype=np.uint8)
    if scales is None:
        scales = np.zeros((n_out, 4 * nb), dtype=np.uint8)
    assert q.dtype == np.uint8 and q.flags.c_contiguous and q.shape[0] == n_out
    assert scales.dtype == np.uint8 and scales.flags.c_contiguous and scales.shape[0] == n_out
    rc = lib().oracle_quantize_act_b128(_ptr(x) if x.size else None, n_rows, cols, x_stride,
                                        _ptr(idx) if idx is not None else None, n_out,
                                        _ptr(q), q.shape[1], _ptr(scales), scales.shape[1])
    if rc != 0:
        raise ValueError("oracle_quantize_act_b128 failed with code %d" % rc)
    sv = scales.view(np.float32) if scales.shape[1] == 4 * nb else scales
    return q, sv
