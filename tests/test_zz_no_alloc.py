"""Plans without allocation (wt_plan_create_noalloc) on the GPU, through the
C ABI: the same bytes as wt_plan_create's plans on the same inputs, call after
call on the device's one scratch array (each call smaller than the one before,
so stale tables of a larger plan would show), and the documented refusals."""
import ctypes

import numpy as np
import pytest
import torch

from bf16_fp8_weight_amd import workloads as W
from gpu_util import assert_images_equal, log, oracle_image_threaded, run_library

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wt():
    from bf16_fp8_weight_amd import wt as _wt
    return _wt


def _noalloc_image(wt, wl, fill=0xA5, replays=2):
    dst = torch.full((wl.dst_bytes,), fill, dtype=torch.uint8, device="cuda")
    h = wt.wt_plan_create_noalloc(wt.task_table(wl), dst.data_ptr(), wl.dst_bytes)
    try:
        s = torch.cuda.current_stream()
        for _ in range(replays):
            wt.wt_prepare(h, s.cuda_stream)
        s.synchronize()
        info = wt.wt_plan_get_info(h)
    finally:
        wt.wt_plan_destroy(h)
    return dst.cpu().numpy(), info


def _workloads():
    # largest first: aligned pairs and fused groups (4 shards), then ragged
    # shapes on the general path (3 shards), then a small fused pair with
    # BF16 copies beside it
    yield "dense_layer_h1024", W.dense_layer_h1024(device="cuda")
    yield "ragged_mix", W.custom([(300, 250), (129, 7), (5, 3000), (257, 1024)], n_shards=3, device="cuda",
                                 dist="t3", seed=11)
    yield "small_fused", W.custom([(64, 72), (200, 72)], n_shards=2, fused=True, device="cuda", seed=12)
    yield "bf16_copies", W.custom([(33, 5), (7, 1)], kind=W.BF16, n_shards=2, device="cuda", seed=13)


def test_noalloc_plans_match_allocating_plans_call_after_call(wt):
    sizes = []
    for name, wl in _workloads():
        log(f"no-allocation plan: {name}, {wl.dst_bytes} destination bytes")
        got, info = _noalloc_image(wt, wl)
        want, winfo = run_library(wl)
        assert info == winfo
        assert_images_equal(got, want, wl)
        assert_images_equal(got, oracle_image_threaded(wl), wl)
        sizes.append(info["n_regular_items"] + info["n_edge_tiles"] + info["n_general_tiles"])
    assert sizes == sorted(sizes, reverse=True) and sizes[-1] < sizes[0]


def test_noalloc_progress_words_count_from_one(wt):
    # the replay counter lives in the scratch array too and starts at 0 for
    # every new plan, whatever the previous plan left there
    wl = W.custom([(256, 256)], n_shards=2, device="cuda", seed=21)
    words = torch.zeros(1, dtype=torch.int64).pin_memory()
    for _ in range(2):
        dst = torch.full((wl.dst_bytes,), 0xA5, dtype=torch.uint8, device="cuda")
        h = wt.wt_plan_create_noalloc(wt.task_table(wl), dst.data_ptr(), wl.dst_bytes)
        try:
            wt.wt_plan_set_progress(h, words.data_ptr(), 1)
            s = torch.cuda.current_stream()
            for _ in range(3):
                wt.wt_prepare(h, s.cuda_stream)
            s.synchronize()
            assert int(words[0]) == 3
        finally:
            wt.wt_plan_destroy(h)
        words.zero_()


def test_noalloc_refusals(wt):
    wl = W.custom([(128, 128)], n_shards=2, device="cuda", seed=31)
    dst = torch.full((wl.dst_bytes,), 0xA5, dtype=torch.uint8, device="cuda")
    h = wt.wt_plan_create_noalloc(wt.task_table(wl), dst.data_ptr(), wl.dst_bytes)
    try:
        # one live plan per device
        with pytest.raises(wt.WtError) as e:
            wt.wt_plan_create_noalloc(wt.task_table(wl), dst.data_ptr(), wl.dst_bytes)
        assert e.value.status == wt.WT_E_STATE
    finally:
        wt.wt_plan_destroy(h)
    # staged writes need staging memory
    opts = wt.wt_plan_options_init()
    opts.dst_write_mode = wt.WT_DST_STAGED
    with pytest.raises(wt.WtError) as e:
        wt.wt_plan_create_noalloc(wt.task_table(wl), dst.data_ptr(), wl.dst_bytes, wt.WT_MEM_DEVICE, opts)
    assert e.value.status == wt.WT_E_INVAL and "staging" in str(e.value)
    # pinned-host shards need staging memory
    hl = W.custom([(64, 128)], n_shards=2, device="cpu", seed=32)
    for o in hl.outputs:
        for p in o.parts:
            p.shards = [s.pin_memory() for s in p.shards]
    hl.shard_mem = "host"
    hdst = torch.full((hl.dst_bytes,), 0xA5, dtype=torch.uint8, device="cuda")
    with pytest.raises(wt.WtError) as e:
        wt.wt_plan_create_noalloc(wt.task_table(hl), hdst.data_ptr(), hl.dst_bytes)
    assert e.value.status == wt.WT_E_INVAL and "staging" in str(e.value)
    # tables above the scratch array's size: one output of 1-row shards,
    # 32 bytes of row-segment table per shard
    n = 540_000
    buf = torch.zeros(n * 8, dtype=torch.bfloat16, device="cuda")
    sh = (wt.wt_shard * n)()
    base = buf.data_ptr()
    for k in range(n):
        sh[k].ptr = base + 16 * k
        sh[k].rows = 1
    tab = wt.TaskTable([{"shards": [(0, 0)], "cols": 8, "dtype": wt.WT_FP8_E4M3FN_B128}])
    tab.arr[0].shards = ctypes.cast(sh, ctypes.POINTER(wt.wt_shard))
    tab.arr[0].n_shards = n
    tiles = (n + 127) // 128
    big_dst = torch.zeros(n * 8 + 4 * tiles + 256, dtype=torch.uint8, device="cuda")
    tab.arr[0].scale_offset = n * 8
    with pytest.raises(wt.WtError) as e:
        wt.wt_plan_create_noalloc(tab, big_dst.data_ptr(), big_dst.numel())
    assert e.value.status == wt.WT_E_NOMEM
    # every refusal released the device's array: a new plan is accepted
    got, _ = _noalloc_image(wt, wl)
    want, _ = run_library(wl)
    assert np.array_equal(got, want)
