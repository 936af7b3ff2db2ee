"""libwt.so on the CPU: it loads, exports every call include/wt.h declares,
and its host-only plan logic (validation, plan shape, pipeline schedule)
behaves as documented. No GPU call is made here."""
import os
import re
import subprocess
import sys

import pytest

from bf16_fp8_weight_amd import workloads as W
from fake_tables import fake_table

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def wt():
    from bf16_fp8_weight_amd import wt as _wt
    return _wt


def _declared():
    src = open(os.path.join(ROOT, "include", "wt.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(wt_[a-z0-9_]+)\s*\(", src)))


def test_exports_match_header(wt):
    names = _declared()
    assert names, "no declarations parsed"
    for n in names:
        assert hasattr(wt.lib, n), n
    assert set(names) == set(wt.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", wt.LIB_PATH], capture_output=True, text=True, check=True).stdout
    syms = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for n in names:
        assert n in syms, n


def test_status_strings(wt):
    assert wt.wt_status_str(0) == "WT_OK"
    for s in range(1, 10):
        assert wt.wt_status_str(s).startswith("WT_E_")


def test_options_defaults(wt):
    o = wt.wt_plan_options_init()
    assert o.watermark_bytes == 512 << 20 and o.dst_write_mode == wt.WT_DST_ZERO_COPY and o.device == -1


def _one(wt, **kw):
    t = {"shards": [(0x10000, 4)], "shard_mem": wt.WT_MEM_DEVICE, "cols": 128,
         "dtype": wt.WT_FP8_E4M3FN_B128, "fusion_group": -1, "dst_offset": 0, "scale_offset": 512}
    t.update(kw)
    return t


def _status(wt, tasks, dst_bytes=4096, kind=None, opts=None):
    tab = wt.TaskTable(tasks)
    try:
        wt.wt_plan_check(tab, dst_bytes, wt.WT_MEM_DEVICE if kind is None else kind, opts)
        return 0
    except wt.WtError as e:
        return e.status


def test_validation_errors(wt):
    E = wt
    assert _status(wt, [_one(wt)]) == 0
    assert _status(wt, []) == E.WT_E_INVAL
    assert _status(wt, [_one(wt, shards=[(0, 4)])]) == E.WT_E_INVAL            # NULL shard with rows
    assert _status(wt, [_one(wt, shards=[(0x10001, 4)])]) == E.WT_E_ALIGN      # odd BF16 pointer
    assert _status(wt, [_one(wt, shards=[(0x10000, -1)])]) == E.WT_E_INVAL     # negative rows
    assert _status(wt, [_one(wt, shards=[(0, 0)])]) == E.WT_E_INVAL            # no rows at all
    assert _status(wt, [_one(wt, cols=0)]) == E.WT_E_INVAL
    assert _status(wt, [_one(wt, dtype=7)]) == E.WT_E_INVAL
    assert _status(wt, [_one(wt, shard_mem=5)]) == E.WT_E_INVAL
    assert _status(wt, [_one(wt, dst_offset=4000)]) == E.WT_E_RANGE            # 512 data bytes past 4096
    assert _status(wt, [_one(wt, scale_offset=4094)]) == E.WT_E_ALIGN
    assert _status(wt, [_one(wt, scale_offset=4096)]) == E.WT_E_RANGE
    assert _status(wt, [_one(wt, scale_offset=100)]) == E.WT_E_OVERLAP         # scale inside the data
    assert _status(wt, [_one(wt), _one(wt, dst_offset=256, scale_offset=1024)]) == E.WT_E_OVERLAP
    assert _status(wt, [_one(wt, dtype=wt.WT_BF16_COPY, dst_offset=1)]) == E.WT_E_ALIGN
    # fusion group members must agree on cols / dtype / memory
    assert _status(wt, [_one(wt, fusion_group=3), _one(wt, fusion_group=3, cols=64)]) == E.WT_E_INVAL
    assert _status(wt, [_one(wt, fusion_group=3), _one(wt, fusion_group=3, shard_mem=wt.WT_MEM_PINNED_HOST)]) == E.WT_E_INVAL
    assert _status(wt, [_one(wt, fusion_group=-2)]) == E.WT_E_INVAL
    assert _status(wt, [_one(wt)], kind=9) == E.WT_E_INVAL
    # pinned-host shards need staging: a watermark below one output's need fails
    o = wt.wt_plan_options_init()
    o.watermark_bytes = 1024
    assert _status(wt, [_one(wt, shard_mem=wt.WT_MEM_PINNED_HOST)], opts=o) == E.WT_E_WATERMARK
    assert "watermark" in wt.wt_plan_last_error(None)


def test_load_hint_range(wt):
    o = wt.wt_plan_options_init()
    assert o.load_hint == wt.WT_LOAD_AUTO
    for h in range(3):
        o.load_hint = h
        assert _status(wt, [_one(wt)], opts=o) == 0
    o.load_hint = 3
    assert _status(wt, [_one(wt)], opts=o) == wt.WT_E_INVAL


def test_max_replays_in_flight_range(wt):
    o = wt.wt_plan_options_init()
    assert o.max_replays_in_flight == 0  # library default
    for v in (1, 2, 8):
        o.max_replays_in_flight = v
        assert _status(wt, [_one(wt)], opts=o) == 0
    o.max_replays_in_flight = 9
    assert _status(wt, [_one(wt)], opts=o) == wt.WT_E_INVAL
    assert "max_replays_in_flight" in wt.wt_plan_last_error(None)


def test_tile_group_option(wt):
    o = wt.wt_plan_options_init()
    assert o.tile_group == wt.WT_GROUP_AUTO
    o.tile_group = 3
    assert _status(wt, [_one(wt)], opts=o) == wt.WT_E_INVAL
    assert "tile_group" in wt.wt_plan_last_error(None)
    # 768 full tiles (one round of workgroups) or fewer: single tiles by default;
    # more: pairs; either forced by the option
    for bands, auto_items in ((24, 24 * 32), (25, 25 * 16)):
        outs = [W.OutputSpec("t", W.FP8, 4096, W._matrix_parts(["w"], [128 * bands], 1))]
        wl = W.Workload("x", outs)
        wl.dst_bytes = W.pack(outs)
        want = {wt.WT_GROUP_AUTO: auto_items, wt.WT_GROUP_SINGLE: bands * 32, wt.WT_GROUP_PAIR: bands * 16}
        for g, n in want.items():
            o = wt.wt_plan_options_init()
            o.tile_group = g
            assert wt.wt_plan_check(fake_table(wt, wl), wl.dst_bytes, opts=o)["n_regular_items"] == n, (bands, g)


def test_fused_group_offsets_from_first_task(wt):
    # the second member's offsets are ignored, so they may be anything
    ok = [_one(wt, fusion_group=1, scale_offset=1024), _one(wt, fusion_group=1, dst_offset=10 ** 9, scale_offset=10 ** 9)]
    info = wt.wt_plan_check(wt.TaskTable(ok), 4096)
    assert info["n_outputs"] == 1 and info["n_tiles"] == 1


@pytest.mark.parametrize("make", [W.dense_layer_h1024, W.kimi_k2_expert_share, W.dense_7b])
def test_plan_shape_matches_workload(wt, make):
    wl = make(materialize=False)
    info = wt.wt_plan_check(fake_table(wt, wl), wl.dst_bytes)
    assert info["n_outputs"] == len(wl.outputs)
    assert info["n_tiles"] == wl.n_tiles
    assert info["input_bytes"] == wl.input_bytes
    assert info["output_bytes"] == wl.output_bytes
    assert info["n_chunks"] == 0 and info["staging_bytes"] == 0
    assert info["n_launches"] == 1  # one batched launch over the whole table


def test_ragged_shapes_use_the_general_kernel(wt):
    wl = W.ragged_stress(materialize=False, n_tensors=64)
    info = wt.wt_plan_check(fake_table(wt, wl), wl.dst_bytes)
    assert info["n_tiles"] == wl.n_tiles
    assert info["n_launches"] == 2  # aligned outputs + general outputs


def _check_schedule(ops, watermark, stages):
    # FIFO per stage: each stage's ops run chunks in increasing order
    for st in stages:
        seq = [o["chunk"] for o in ops if o["stage"] == st and o["chunk"] >= 0]
        assert seq == sorted(seq) and len(seq) == len(set(seq))
    # worst case (nothing completes unless a wait forces it): at each
    # admission the live chunks' slots are disjoint and within the watermark
    first = {}
    for o in ops:
        first.setdefault(o["chunk"], o)
    released = -1
    slots = {}
    for c in sorted(k for k in first if k >= 0):
        o = first[c]
        if o["wait_chunk"] >= 0:
            assert o["wait_chunk"] < c
            released = max(released, o["wait_chunk"])
        slots[c] = (o["staging_offset"], o["staging_offset"] + o["staging_bytes"])
        live = [slots[k] for k in slots if released < k <= c]
        assert sum(b - a for a, b in live) <= watermark
        assert all(b <= watermark for _, b in live)
        live.sort()
        for (a0, b0), (a1, b1) in zip(live, live[1:]):
            assert b0 <= a1, "live staging slots overlap"


@pytest.mark.parametrize("watermark_mb", [160, 256, 1024])
def test_pipeline_schedule_host_shards(wt, watermark_mb):
    wl = W.mla_many_small(materialize=False)
    o = wt.wt_plan_options_init()
    o.watermark_bytes = watermark_mb << 20
    tab = fake_table(wt, wl, align=16)
    info = wt.wt_plan_check(tab, wl.dst_bytes, opts=o)
    ops = wt.wt_plan_schedule(tab, wl.dst_bytes, opts=o)
    assert info["n_chunks"] == max(op["chunk"] for op in ops) + 1
    assert info["staging_bytes"] <= o.watermark_bytes
    assert sum(op["bytes"] for op in ops if op["stage"] == 0) == wl.input_bytes
    assert sum(op["bytes"] for op in ops if op["stage"] == 1) == wl.input_bytes
    _check_schedule(ops, o.watermark_bytes, stages=(0, 1))
    # contiguous host shards merge into one copy per chunk
    assert info["n_h2d_copies"] == info["n_chunks"]


def test_pipeline_schedule_staged_mode(wt):
    wl = W.dense_layer_h1024(materialize=False)
    o = wt.wt_plan_options_init()
    o.dst_write_mode = wt.WT_DST_STAGED
    o.watermark_bytes = 16 << 20
    tab = fake_table(wt, wl)
    ops = wt.wt_plan_schedule(tab, wl.dst_bytes, opts=o)
    assert [op["stage"] for op in ops] == [1, 2] * (len(ops) // 2)
    assert sum(op["bytes"] for op in ops if op["stage"] == 2) == wl.output_bytes
    _check_schedule(ops, o.watermark_bytes, stages=(1, 2))


def test_gapped_host_shards_copy_per_run(wt):
    wl = W.custom([(300, 256), (64, 128)], n_shards=4, device="cpu")
    o = wt.wt_plan_options_init()
    tab = fake_table(wt, wl, gap=512, host=True)
    info = wt.wt_plan_check(tab, wl.dst_bytes, opts=o)
    assert info["n_h2d_copies"] == 8  # no merging across gaps


def test_completion_units(wt):
    # device-resident zero-copy: the one launch is the one unit
    wl = W.dense_layer_h1024(materialize=False)
    assert wt.wt_plan_check(fake_table(wt, wl), wl.dst_bytes)["n_units"] == 1
    # pinned-host shards: one unit per chunk
    wl = W.mla_many_small(materialize=False, layers=1, n_small=300, host=True)
    o = wt.wt_plan_options_init()
    o.chunk_bytes = 8 << 20
    i = wt.wt_plan_check(fake_table(wt, wl), wl.dst_bytes, wt.WT_MEM_PINNED_HOST, o)
    assert i["n_units"] == i["n_chunks"] > 1
    # mixed: device-resident outputs launch first as unit 0, then the chunks
    wl = W.mla_many_small(materialize=False, layers=1, n_small=300, host=True)
    tab = fake_table(wt, wl).as_dicts()
    for t in tab[:3]:
        t["shard_mem"] = wt.WT_MEM_DEVICE
    i = wt.wt_plan_check(wt.TaskTable(tab), wl.dst_bytes, wt.WT_MEM_PINNED_HOST, o)
    assert i["n_units"] == i["n_chunks"] + 1


def test_progress_wait_on_the_host(wt):
    import ctypes
    import threading
    import time

    w = (ctypes.c_uint64 * 2)(7, 0)
    a = ctypes.addressof(w)
    assert wt.wt_progress_wait(a, 7, 0) and wt.wt_progress_wait(a, 3, 10)
    t0 = time.perf_counter()
    assert not wt.wt_progress_wait(a, 8, 20 * 10**6)
    assert 0.015 < time.perf_counter() - t0 < 5
    with pytest.raises(wt.WtError):
        wt.wt_progress_wait(0, 1, 10)

    def later():
        time.sleep(0.05)
        w[1] = 1
    th = threading.Thread(target=later)
    th.start()
    assert wt.wt_progress_wait(a + 8, 1, 10 * 10**9)
    th.join()


def test_default_chunking_bounds_chunk_count(wt):
    # about 16 chunks per replay by default, at most watermark / 2 bytes each;
    # an explicit chunk size is honoured
    wl = W.mla_many_small(materialize=False)
    tab = fake_table(wt, wl)
    i = wt.wt_plan_check(tab, wl.dst_bytes, wt.WT_MEM_DEVICE)
    assert 12 <= i["n_chunks"] <= 24
    o = wt.wt_plan_options_init()
    o.chunk_bytes = 8 << 20
    assert wt.wt_plan_check(tab, wl.dst_bytes, wt.WT_MEM_DEVICE, o)["n_chunks"] > 40
    o = wt.wt_plan_options_init()
    o.watermark_bytes = 1 << 30
    ops = wt.wt_plan_schedule(tab, wl.dst_bytes, opts=o)
    assert max(op["staging_bytes"] for op in ops if op["stage"] == 0) <= (1 << 29) + (1 << 20)


def test_default_chunk_leaves_a_slot_per_busy_stage(wt):
    # 64 host-resident 2048 x 4096 tensors (16 MiB each) under a 128 MiB
    # watermark: when outputs are staged too, three stages hold staging at once
    # and a default chunk takes at most a third of the watermark; with zero-copy
    # outputs two stages do and the bound is half
    rows, cols, n = 2048, 4096, 64
    data, scales = rows * cols, (rows // 128) * (cols // 128) * 4
    tasks = [{"shards": [(0x7F0000000000 + i * 2 * rows * cols, rows)], "shard_mem": wt.WT_MEM_PINNED_HOST,
              "cols": cols, "dtype": wt.WT_FP8_E4M3FN_B128, "fusion_group": -1,
              "dst_offset": i * data, "scale_offset": n * data + i * scales} for i in range(n)]
    tab = wt.TaskTable(tasks)
    wm = 128 << 20
    slots = {}
    for mode in (wt.WT_DST_STAGED, wt.WT_DST_ZERO_COPY):
        o = wt.wt_plan_options_init()
        o.watermark_bytes = wm
        o.dst_write_mode = mode
        ops = wt.wt_plan_schedule(tab, n * (data + scales), opts=o)
        slots[mode] = max(op["staging_bytes"] for op in ops if op["stage"] == 0)
    assert slots[wt.WT_DST_STAGED] <= wm // 3
    assert wm // 3 < slots[wt.WT_DST_ZERO_COPY] <= wm // 2


def test_plain_c_program_uses_the_abi(wt, tmp_path):
    # the header compiles as C99 and a C program linked against libwt.so drives
    # the host-only entry points without the Python binding
    exe = tmp_path / "c_abi_check"
    libdir = os.path.dirname(wt.LIB_PATH)
    src = os.path.join(ROOT, "tests", "c_abi", "c_abi_check.c")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    src, "-o", str(exe), f"-L{libdir}", f"-l:{os.path.basename(wt.LIB_PATH)}",
                    f"-Wl,-rpath,{libdir}"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "c abi ok" in r.stdout, r.stdout + r.stderr


def test_work_item_counts(wt):
    # full single-shard tiles go in pairs on the aligned path; tiles across shards are edge tiles;
    # ragged outputs go to the general path
    wl = W.kimi_k2_expert_share(materialize=False)
    i = wt.wt_plan_check(fake_table(wt, wl), wl.dst_bytes)
    assert (i["n_regular_items"], i["n_edge_tiles"], i["n_general_tiles"]) == (wl.n_tiles // 2, 0, 0)
    outs = [W.OutputSpec("t", W.FP8, 384, W._matrix_parts(["w"], [1536], 8))]  # 192-row shards, 3 tiles per band
    wl = W.Workload("x", outs)
    wl.dst_bytes = W.pack(outs)
    o = wt.wt_plan_options_init()
    o.tile_group = wt.WT_GROUP_PAIR
    i = wt.wt_plan_check(fake_table(wt, wl), wl.dst_bytes, opts=o)
    # 12 bands: 8 of them inside one shard (a pair + a single each), 4 straddle a shard boundary
    assert (i["n_regular_items"], i["n_edge_tiles"], i["n_general_tiles"]) == (16, 12, 0)
    # 36 tiles fit in one round of workgroups: by default every full tile is its own item
    i = wt.wt_plan_check(fake_table(wt, wl), wl.dst_bytes)
    assert (i["n_regular_items"], i["n_edge_tiles"], i["n_general_tiles"]) == (24, 12, 0)
    wl = W.ragged_stress(materialize=False, n_tensors=16)
    i = wt.wt_plan_check(fake_table(wt, wl), wl.dst_bytes)
    assert i["n_general_tiles"] > 0
    assert i["n_regular_items"] * 2 + i["n_edge_tiles"] + i["n_general_tiles"] >= i["n_tiles"]


def test_binding_fails_loudly_without_the_library(tmp_path):
    # no fallback of any kind: importing the binding with the library missing raises
    env = dict(os.environ, WT_LIB=str(tmp_path / "missing" / "libwt.so"))
    r = subprocess.run([sys.executable, "-c", "import bf16_fp8_weight_amd.wt"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT, env=env)
    assert r.returncode != 0 and "ImportError" in r.stderr


def test_plan_keeps_shards_and_destination_alive(wt, monkeypatch):
    # a Plan holds raw shard and destination addresses: the workload's shard
    # tensors and the destination must live as long as the plan does, even
    # when the caller drops its own references
    import gc
    import weakref

    import torch

    wl = W.custom([(5, 7), (3, 7)], device="cpu")
    shard_refs = [weakref.ref(s) for o in wl.outputs for p in o.parts for s in p.shards]
    dst = torch.empty(wl.dst_bytes, dtype=torch.uint8)
    dst_ref = weakref.ref(dst)
    destroyed = []
    monkeypatch.setattr(wt, "wt_plan_create", lambda *a, **k: 12345)
    monkeypatch.setattr(wt, "wt_plan_destroy", lambda h: destroyed.append(h))
    plan = wt.Plan(wl, dst)
    del wl, dst
    gc.collect()
    assert all(r() is not None for r in shard_refs) and dst_ref() is not None
    plan.close()
    assert destroyed == [12345]
    gc.collect()
    assert all(r() is None for r in shard_refs) and dst_ref() is None
