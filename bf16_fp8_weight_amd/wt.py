"""ctypes binding of libwt.so (C ABI in include/wt.h), same names as the C calls.

Argument marshalling only: every step of the preparation runs in the
library's HIP kernels. PyTorch is used by callers for device memory and
streams; this module passes raw addresses. Importing it raises if libwt.so has
not been built, so no caller can silently run without the GPU library.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
# WT_LIB selects another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("WT_LIB") or os.path.join(PKG, "libwt.so")

WT_OK = 0
(WT_E_INVAL, WT_E_RANGE, WT_E_OVERLAP, WT_E_ALIGN, WT_E_NOMEM, WT_E_HIP, WT_E_WATERMARK, WT_E_STATE,
 WT_E_TIMEOUT) = range(1, 10)
WT_FP8_E4M3FN_B128 = 0
WT_BF16_COPY = 1
WT_MEM_DEVICE = 0
WT_MEM_PINNED_HOST = 1
WT_DST_ZERO_COPY = 0
WT_DST_STAGED = 1
WT_LOAD_AUTO, WT_LOAD_PLAIN, WT_LOAD_STREAM = range(3)
WT_GROUP_AUTO, WT_GROUP_SINGLE, WT_GROUP_PAIR = range(3)

EXPORTS = [
    "wt_plan_options_init", "wt_plan_check", "wt_plan_schedule", "wt_plan_create", "wt_prepare",
    "wt_plan_get_info", "wt_plan_destroy", "wt_status_str", "wt_plan_last_error",
    "wt_quantize_domain", "wt_cast_f32_range",
    "wt_schedule_build", "wt_schedule_info", "wt_schedule_output", "wt_schedule_tasks", "wt_schedule_destroy",
    "wt_plan_set_progress", "wt_plan_task_unit", "wt_progress_wait", "wt_quantize_act_b128",
    "wt_plan_create_noalloc",
]


class wt_shard(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("rows", ctypes.c_int64)]


class wt_task(ctypes.Structure):
    _fields_ = [
        ("shards", ctypes.POINTER(wt_shard)),
        ("n_shards", ctypes.c_int32),
        ("shard_mem", ctypes.c_int32),
        ("cols", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("fusion_group", ctypes.c_int32),
        ("dst_offset", ctypes.c_uint64),
        ("scale_offset", ctypes.c_uint64),
    ]


class wt_plan_options(ctypes.Structure):
    _fields_ = [
        ("watermark_bytes", ctypes.c_uint64),
        ("chunk_bytes", ctypes.c_uint64),
        ("dst_write_mode", ctypes.c_int32),
        ("device", ctypes.c_int32),
        ("load_hint", ctypes.c_uint32),
        ("max_replays_in_flight", ctypes.c_uint32),
        ("tile_group", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32 * 3),
    ]


class wt_plan_info(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "n_tasks", "n_outputs", "n_fp8_outputs", "n_copy_outputs", "n_tiles", "input_bytes", "output_bytes",
        "n_launches", "n_chunks", "n_h2d_copies", "n_dst_copies", "staging_bytes", "n_units", "n_regular_items",
        "n_edge_tiles", "n_general_tiles")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_ if n != "reserved"}


class wt_sched_op(ctypes.Structure):
    _fields_ = [
        ("stage", ctypes.c_int32),
        ("chunk", ctypes.c_int32),
        ("wait_chunk", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("bytes", ctypes.c_int64),
        ("staging_offset", ctypes.c_int64),
        ("staging_bytes", ctypes.c_int64),
    ]


class wt_param_meta(ctypes.Structure):
    _fields_ = [
        ("name", ctypes.c_char_p),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("n_shards", ctypes.c_int32),
        ("shard_mem", ctypes.c_int32),
        ("shard_ptrs", ctypes.POINTER(ctypes.c_void_p)),
    ]


class wt_dst_meta(ctypes.Structure):
    _fields_ = [
        ("name", ctypes.c_char_p),
        ("components", ctypes.POINTER(ctypes.c_char_p)),
        ("n_components", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


class wt_schedule_options(ctypes.Structure):
    _fields_ = [("align", ctypes.c_uint64), ("n_sources", ctypes.c_int32), ("reserved", ctypes.c_int32 * 5)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libwt.so not found at {LIB_PATH}: build it first (python -m bf16_fp8_weight_amd.build or "
            "__graft_entry__.build()); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    P = ctypes.POINTER
    L.wt_plan_options_init.restype = None
    L.wt_plan_options_init.argtypes = [P(wt_plan_options)]
    L.wt_plan_check.restype = ctypes.c_int
    L.wt_plan_check.argtypes = [P(wt_task), sz, sz, i32, P(wt_plan_options), P(wt_plan_info)]
    L.wt_plan_schedule.restype = ctypes.c_int
    L.wt_plan_schedule.argtypes = [P(wt_task), sz, sz, i32, P(wt_plan_options), P(wt_sched_op), sz, P(sz)]
    L.wt_plan_create.restype = ctypes.c_int
    L.wt_plan_create.argtypes = [P(wt_task), sz, vp, sz, i32, P(wt_plan_options), P(vp)]
    L.wt_plan_create_noalloc.restype = ctypes.c_int
    L.wt_plan_create_noalloc.argtypes = [P(wt_task), sz, vp, sz, i32, P(wt_plan_options), P(vp)]
    L.wt_prepare.restype = ctypes.c_int
    L.wt_prepare.argtypes = [vp, vp]
    L.wt_plan_get_info.restype = ctypes.c_int
    L.wt_plan_get_info.argtypes = [vp, P(wt_plan_info)]
    L.wt_plan_destroy.restype = None
    L.wt_plan_destroy.argtypes = [vp]
    L.wt_status_str.restype = ctypes.c_char_p
    L.wt_status_str.argtypes = [ctypes.c_int]
    L.wt_plan_last_error.restype = ctypes.c_char_p
    L.wt_plan_last_error.argtypes = [vp]
    L.wt_quantize_domain.restype = ctypes.c_int
    L.wt_quantize_domain.argtypes = [vp, i64, i32, vp, vp]
    L.wt_cast_f32_range.restype = ctypes.c_int
    L.wt_cast_f32_range.argtypes = [ctypes.c_uint32, ctypes.c_uint64, vp, vp]
    L.wt_schedule_build.restype = ctypes.c_int
    L.wt_schedule_build.argtypes = [P(wt_param_meta), sz, P(wt_dst_meta), sz, P(wt_schedule_options), P(vp)]
    L.wt_schedule_info.restype = ctypes.c_int
    L.wt_schedule_info.argtypes = [vp, P(sz), P(sz), P(ctypes.c_uint64), P(sz)]
    L.wt_schedule_output.restype = ctypes.c_int
    L.wt_schedule_output.argtypes = [vp, sz, P(ctypes.c_uint64), P(ctypes.c_uint64), P(i32), P(ctypes.c_uint64)]
    L.wt_schedule_tasks.restype = ctypes.c_int
    L.wt_schedule_tasks.argtypes = [vp, i32, P(wt_task), sz, P(wt_shard), sz, P(sz), P(sz)]
    L.wt_schedule_destroy.restype = None
    L.wt_schedule_destroy.argtypes = [vp]
    L.wt_plan_set_progress.restype = ctypes.c_int
    L.wt_plan_set_progress.argtypes = [vp, vp, sz]
    L.wt_plan_task_unit.restype = ctypes.c_int
    L.wt_plan_task_unit.argtypes = [vp, sz, P(i32)]
    L.wt_quantize_act_b128.restype = ctypes.c_int
    L.wt_quantize_act_b128.argtypes = [vp, i64, i64, i64, vp, i64, vp, i64, vp, i64, vp]
    L.wt_progress_wait.restype = ctypes.c_int
    L.wt_progress_wait.argtypes = [vp, ctypes.c_uint64, ctypes.c_uint64]
    return L


lib = _load()


class WtError(RuntimeError):
    def __init__(self, status: int, detail: str = ""):
        self.status = status
        msg = lib.wt_status_str(status).decode()
        super().__init__(msg + (f": {detail}" if detail else ""))


def _check(st: int, plan=None) -> None:
    if st != WT_OK:
        d = lib.wt_plan_last_error(plan)
        raise WtError(st, d.decode() if d else "")


# ------------------------------------------------------------- same-name calls
def wt_plan_options_init() -> wt_plan_options:
    o = wt_plan_options()
    lib.wt_plan_options_init(ctypes.byref(o))
    return o


class TaskTable:
    """A ctypes task table plus the shard arrays it points to (kept alive)."""

    def __init__(self, tasks: Sequence[dict]):
        self._shards: List = []
        self.arr = (wt_task * max(1, len(tasks)))()
        self.n = len(tasks)
        for i, t in enumerate(tasks):
            sh = (wt_shard * max(1, len(t["shards"])))()
            for k, (ptr, rows) in enumerate(t["shards"]):
                sh[k].ptr = ptr or None
                sh[k].rows = rows
            self._shards.append(sh)
            a = self.arr[i]
            a.shards = ctypes.cast(sh, ctypes.POINTER(wt_shard)) if t["shards"] else None
            a.n_shards = len(t["shards"])
            a.shard_mem = t.get("shard_mem", WT_MEM_DEVICE)
            a.cols = t["cols"]
            a.dtype = t["dtype"]
            a.fusion_group = t.get("fusion_group", -1)
            a.dst_offset = t.get("dst_offset", 0)
            a.scale_offset = t.get("scale_offset", 0)

    def as_dicts(self) -> List[dict]:
        """The table read back in the form the constructor takes."""
        out = []
        for i in range(self.n):
            a = self.arr[i]
            out.append({
                "shards": [(a.shards[k].ptr or 0, a.shards[k].rows) for k in range(a.n_shards)],
                "shard_mem": a.shard_mem, "cols": a.cols, "dtype": a.dtype, "fusion_group": a.fusion_group,
                "dst_offset": a.dst_offset, "scale_offset": a.scale_offset,
            })
        return out


def wt_plan_check(table: TaskTable, dst_bytes: int, dst_kind: int = WT_MEM_DEVICE,
                  opts: Optional[wt_plan_options] = None) -> dict:
    info = wt_plan_info()
    _check(lib.wt_plan_check(table.arr, table.n, dst_bytes, dst_kind, ctypes.byref(opts) if opts else None,
                             ctypes.byref(info)))
    return info.as_dict()


def wt_plan_schedule(table: TaskTable, dst_bytes: int, dst_kind: int = WT_MEM_DEVICE,
                     opts: Optional[wt_plan_options] = None) -> List[dict]:
    n = ctypes.c_size_t(0)
    po = ctypes.byref(opts) if opts else None
    _check(lib.wt_plan_schedule(table.arr, table.n, dst_bytes, dst_kind, po, None, 0, ctypes.byref(n)))
    ops = (wt_sched_op * max(1, n.value))()
    _check(lib.wt_plan_schedule(table.arr, table.n, dst_bytes, dst_kind, po, ops, n.value, ctypes.byref(n)))
    return [{f: int(getattr(ops[i], f)) for f, _ in wt_sched_op._fields_ if f != "reserved"} for i in range(n.value)]


def wt_plan_create(table: TaskTable, dst_ptr: int, dst_bytes: int, dst_kind: int = WT_MEM_DEVICE,
                   opts: Optional[wt_plan_options] = None) -> int:
    out = ctypes.c_void_p(0)
    _check(lib.wt_plan_create(table.arr, table.n, dst_ptr, dst_bytes, dst_kind,
                              ctypes.byref(opts) if opts else None, ctypes.byref(out)))
    return out.value


def wt_plan_create_noalloc(table: TaskTable, dst_ptr: int, dst_bytes: int, dst_kind: int = WT_MEM_DEVICE,
                           opts: Optional[wt_plan_options] = None) -> int:
    out = ctypes.c_void_p(0)
    _check(lib.wt_plan_create_noalloc(table.arr, table.n, dst_ptr, dst_bytes, dst_kind,
                                      ctypes.byref(opts) if opts else None, ctypes.byref(out)))
    return out.value


def wt_prepare(plan: int, stream: int = 0) -> None:
    _check(lib.wt_prepare(plan, stream or None), plan)


def wt_plan_get_info(plan: int) -> dict:
    info = wt_plan_info()
    _check(lib.wt_plan_get_info(plan, ctypes.byref(info)), plan)
    return info.as_dict()


def wt_plan_set_progress(plan: int, words: int, n_words: int) -> None:
    """words: address of n_words uint64 in pinned host memory (0 detaches)."""
    _check(lib.wt_plan_set_progress(plan, words or None, n_words), plan)


def wt_plan_task_unit(plan: int, task: int) -> int:
    u = ctypes.c_int32()
    _check(lib.wt_plan_task_unit(plan, task, ctypes.byref(u)), plan)
    return u.value


def wt_progress_wait(word: int, target: int, timeout_ns: int) -> bool:
    """True once *word >= target, False on timeout."""
    st = lib.wt_progress_wait(word or None, target, timeout_ns)
    if st == WT_E_TIMEOUT:
        return False
    _check(st)
    return True


def wt_quantize_act_b128(x: int, n_rows: int, cols: int, x_row_stride: int, row_index: int, n_out: int, q: int,
                         q_row_stride: int, scales: int, scale_row_stride: int, stream: int = 0) -> None:
    """Addresses as integers (0 = NULL); see include/wt.h."""
    _check(lib.wt_quantize_act_b128(x or None, n_rows, cols, x_row_stride, row_index or None, n_out, q or None,
                                    q_row_stride, scales or None, scale_row_stride, stream or None))


def wt_plan_destroy(plan: int) -> None:
    lib.wt_plan_destroy(plan)


def wt_status_str(status: int) -> str:
    return lib.wt_status_str(status).decode()


def wt_plan_last_error(plan: Optional[int] = None) -> str:
    r = lib.wt_plan_last_error(plan)
    return r.decode() if r else ""


def wt_quantize_domain(amax_bits_ptr: int, n_amax: int, path: int, out_ptr: int, stream: int = 0) -> None:
    _check(lib.wt_quantize_domain(amax_bits_ptr, n_amax, path, out_ptr, stream or None))


def wt_cast_f32_range(first: int, count: int, out_ptr: int, stream: int = 0) -> None:
    _check(lib.wt_cast_f32_range(first, count, out_ptr, stream or None))


# ------------------------------------------------------------- schedule builder
class Schedule:
    """Result of wt_schedule_build; the same calls as methods.

    params: dicts {name, rows, cols, n_shards, shard_mem?, shard_ptrs?}
    dsts:   dicts {name, components: [names], dtype}
    """

    def __init__(self, params, dsts, align: int = 256, n_sources: int = 1):
        self._keep = []
        pa = (wt_param_meta * max(1, len(params)))()
        for i, p in enumerate(params):
            nm = p["name"].encode()
            self._keep.append(nm)
            pa[i].name = nm
            pa[i].rows, pa[i].cols = p["rows"], p["cols"]
            pa[i].n_shards = p["n_shards"]
            pa[i].shard_mem = p.get("shard_mem", WT_MEM_DEVICE)
            if p.get("shard_ptrs") is not None:
                arr = (ctypes.c_void_p * p["n_shards"])(*[x or None for x in p["shard_ptrs"]])
                self._keep.append(arr)
                pa[i].shard_ptrs = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
        da = (wt_dst_meta * max(1, len(dsts)))()
        for i, d in enumerate(dsts):
            nm = d["name"].encode()
            comps = (ctypes.c_char_p * len(d["components"]))(*[c.encode() for c in d["components"]])
            self._keep += [nm, comps]
            da[i].name = nm
            da[i].components = ctypes.cast(comps, ctypes.POINTER(ctypes.c_char_p))
            da[i].n_components = len(d["components"])
            da[i].dtype = d["dtype"]
        o = wt_schedule_options()
        o.align, o.n_sources = align, n_sources
        h = ctypes.c_void_p(0)
        _check(lib.wt_schedule_build(pa, len(params), da, len(dsts), ctypes.byref(o), ctypes.byref(h)))
        self.handle = h.value
        self.n_dsts = len(dsts)

    def info(self) -> dict:
        nt, ns, nu = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
        db = ctypes.c_uint64()
        _check(lib.wt_schedule_info(self.handle, ctypes.byref(nt), ctypes.byref(ns), ctypes.byref(db), ctypes.byref(nu)))
        return {"n_tasks": nt.value, "n_shards": ns.value, "dst_bytes": db.value, "n_unused_params": nu.value}

    def output(self, i: int) -> dict:
        do, so, ib = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
        src = ctypes.c_int32()
        _check(lib.wt_schedule_output(self.handle, i, ctypes.byref(do), ctypes.byref(so), ctypes.byref(src),
                                      ctypes.byref(ib)))
        return {"dst_offset": do.value, "scale_offset": so.value, "source": src.value, "input_bytes": ib.value}

    def tasks(self, source: int = -1) -> TaskTable:
        nt, ns = ctypes.c_size_t(), ctypes.c_size_t()
        st = lib.wt_schedule_tasks(self.handle, source, None, 0, None, 0, ctypes.byref(nt), ctypes.byref(ns))
        if st not in (WT_OK, WT_E_RANGE):
            _check(st)
        tab = TaskTable([])
        tab.arr = (wt_task * max(1, nt.value))()
        sh = (wt_shard * max(1, ns.value))()
        _check(lib.wt_schedule_tasks(self.handle, source, tab.arr, nt.value, sh, ns.value, ctypes.byref(nt),
                                     ctypes.byref(ns)))
        tab.n = nt.value
        tab._shards = [sh]
        return tab

    def close(self) -> None:
        if getattr(self, "handle", 0):
            lib.wt_schedule_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------------- workload glue
def task_table(wl, group_base: int = 0) -> TaskTable:
    """Task table for a bf16_fp8_weight_amd.workloads.Workload: one task per
    component, components of a fused output share a fusion group."""
    from . import workloads as W

    tasks = []
    for oi, o in enumerate(wl.outputs):
        fused = len(o.parts) > 1
        for p in o.parts:
            tasks.append({
                "shards": [(s.data_ptr() if r else 0, r) for s, r in zip(p.shards, p.shard_rows)],
                "shard_mem": WT_MEM_PINNED_HOST if wl.shard_mem == "host" else WT_MEM_DEVICE,
                "cols": o.cols,
                "dtype": WT_FP8_E4M3FN_B128 if o.kind == W.FP8 else WT_BF16_COPY,
                "fusion_group": group_base + oi if fused else -1,
                "dst_offset": o.dst_offset,
                "scale_offset": o.scale_offset,
            })
    return TaskTable(tasks)


class Plan:
    """Owns a wt_plan handle for a workload and a destination tensor.

    The plan holds the shards' and the destination's addresses, so it keeps
    the workload (and with it every shard tensor and the pinned arena) and the
    destination tensor alive until it is closed."""

    def __init__(self, wl, dst, dst_kind: int = WT_MEM_DEVICE, opts: Optional[wt_plan_options] = None):
        self.wl = wl
        self.table = task_table(wl)
        self.dst = dst
        self.handle = wt_plan_create(self.table, dst.data_ptr(), dst.numel() * dst.element_size(), dst_kind, opts)

    def prepare(self, stream: int = 0) -> None:
        wt_prepare(self.handle, stream)

    def info(self) -> dict:
        return wt_plan_get_info(self.handle)

    def close(self) -> None:
        if self.handle:
            wt_plan_destroy(self.handle)
            self.handle = 0
        self.wl = None
        self.dst = None

    def __enter__(self) -> "Plan":
        return self

    def __exit__(self, *exc) -> None:
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
