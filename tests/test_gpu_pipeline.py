"""The three-stage pipeline (host-to-device copy, prepare, destination copy)
and destination modes, against the oracle; plus create-time memory checks.
Marked gpu."""
import numpy as np
import pytest
import torch

from bf16_fp8_weight_amd import workloads as W
from gpu_util import Timer, assert_images_equal, log, oracle_image_threaded, run_library

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wt():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from bf16_fp8_weight_amd import wt as _wt
    return _wt


@pytest.fixture(scope="module")
def mla():
    wl = W.mla_many_small(device="cuda")  # shards in one pinned host arena
    with Timer("oracle"):
        want = oracle_image_threaded(wl)
    return wl, want


@pytest.mark.parametrize("watermark_mb,chunk_mb", [(256, 0), (160, 8), (1024, 64)])
def test_mla_pinned_host_shards(wt, mla, watermark_mb, chunk_mb):
    wl, want = mla
    o = wt.wt_plan_options_init()
    o.watermark_bytes = watermark_mb << 20
    o.chunk_bytes = chunk_mb << 20
    got, info = run_library(wl, opts=o)
    log(f"  watermark {watermark_mb} MiB: {info['n_chunks']} chunks, {info['n_h2d_copies']} H2D copies, "
        f"{info['n_launches']} launches, staging {info['staging_bytes'] >> 20} MiB")
    assert info["staging_bytes"] <= o.watermark_bytes
    assert_images_equal(got, want, wl)


def test_mla_staged_to_pinned_host_dst(wt, mla):
    wl, want = mla
    o = wt.wt_plan_options_init()
    o.dst_write_mode = wt.WT_DST_STAGED
    got, info = run_library(wl, opts=o, dst_kind=wt.WT_MEM_PINNED_HOST)
    assert info["n_dst_copies"] > 0
    assert_images_equal(got, want, wl)


def test_zero_copy_into_pinned_host_dst(wt):
    wl = W.dense_layer_h1024(device="cuda")
    got, _ = run_library(wl, dst_kind=wt.WT_MEM_PINNED_HOST)
    assert_images_equal(got, oracle_image_threaded(wl), wl)


def test_staged_device_resident(wt):
    wl = W.custom([(300, 512), (64, 64), (1, 300), (129, 17), (4096, 1024)], n_shards=3, device="cuda")
    o = wt.wt_plan_options_init()
    o.dst_write_mode = wt.WT_DST_STAGED
    o.watermark_bytes = 12 << 20
    o.chunk_bytes = 1 << 20
    got, info = run_library(wl, opts=o)
    assert info["n_chunks"] > 1
    assert_images_equal(got, oracle_image_threaded(wl), wl)


def test_repeated_replays_on_one_stream(wt):
    # back-to-back replays without a host sync: the next replay's copies must
    # wait for the previous one's use of the staging ring
    wl = W.mla_many_small(device="cuda", layers=2, n_small=200)
    from bf16_fp8_weight_amd import wt as _wt
    o = _wt.wt_plan_options_init()
    o.watermark_bytes = 160 << 20  # above the largest output (o: 117 MB of BF16)
    o.chunk_bytes = 4 << 20
    dst = torch.full((wl.dst_bytes,), 0xA5, dtype=torch.uint8, device="cuda")
    h = _wt.wt_plan_create(_wt.task_table(wl), dst.data_ptr(), wl.dst_bytes, _wt.WT_MEM_DEVICE, o)
    try:
        s = torch.cuda.current_stream()
        for _ in range(4):
            _wt.wt_prepare(h, s.cuda_stream)
        s.synchronize()
    finally:
        _wt.wt_plan_destroy(h)
    assert_images_equal(dst.cpu().numpy(), oracle_image_threaded(wl), wl)


@pytest.mark.parametrize("depth", [1, 2, 3])
def test_replays_in_flight_keep_order(wt, depth):
    # a staged plan over device-resident shards (pipelined), replayed back to
    # back with max_replays_in_flight = depth; before each replay after the
    # first a stream-ordered kernel negates every shard, so replay r reads
    # (-1)^r x. Six negations bring the inputs back to x, which the last replay
    # read: the final image is the oracle's unless replays overlap or reorder
    wl = W.custom([(300, 512), (129, 17), (1000, 1024), (64, 64), (200, 300), (77, 129), (500, 256), (33, 1000)],
                  n_shards=3, device="cuda")
    o = wt.wt_plan_options_init()
    o.dst_write_mode = wt.WT_DST_STAGED
    o.watermark_bytes = 3 << 20  # the ring wraps, so slots are reused within and across replays
    o.chunk_bytes = 128 << 10
    o.max_replays_in_flight = depth
    dst = torch.full((wl.dst_bytes,), 0xA5, dtype=torch.uint8, device="cuda")
    h = wt.wt_plan_create(wt.task_table(wl), dst.data_ptr(), wl.dst_bytes, wt.WT_MEM_DEVICE, o)
    try:
        assert wt.wt_plan_get_info(h)["n_chunks"] > 2
        s = torch.cuda.current_stream()
        for r in range(7):
            if r:
                for out in wl.outputs:
                    for part in out.parts:
                        for sh in part.shards:
                            sh.neg_()
            wt.wt_prepare(h, s.cuda_stream)
        s.synchronize()
    finally:
        wt.wt_plan_destroy(h)
    assert_images_equal(dst.cpu().numpy(), oracle_image_threaded(wl), wl)


def test_create_rejects_bad_memory(wt):
    wl = W.custom([(128, 128)], n_shards=2, device="cuda")
    dst = torch.zeros(wl.dst_bytes, dtype=torch.uint8, device="cuda")
    # pageable host memory given as the destination region
    host = torch.zeros(wl.dst_bytes, dtype=torch.uint8)
    with pytest.raises(wt.WtError) as e:
        wt.wt_plan_create(wt.task_table(wl), host.data_ptr(), wl.dst_bytes)
    assert e.value.status == wt.WT_E_INVAL
    # destination size larger than its allocation
    with pytest.raises(wt.WtError) as e:
        wt.wt_plan_create(wt.task_table(wl), dst.data_ptr(), wl.dst_bytes + (64 << 20))
    assert e.value.status in (wt.WT_E_RANGE,)
    # device shards declared as pinned host
    tab = wt.task_table(wl)
    for i in range(tab.n):
        tab.arr[i].shard_mem = wt.WT_MEM_PINNED_HOST
    with pytest.raises(wt.WtError) as e:
        wt.wt_plan_create(tab, dst.data_ptr(), wl.dst_bytes)
    assert e.value.status == wt.WT_E_INVAL


def test_create_rejects_pinned_host_ranges_past_their_allocation(wt):
    # pinned-host destination and pinned-host shards are checked against the
    # extent of their allocation like device memory: refused at create time,
    # before any kernel runs. Two 1 MiB pinned allocations of exactly known
    # size from the HIP runtime.
    import ctypes

    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipHostMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t, ctypes.c_uint]
    hip.hipHostFree.argtypes = [ctypes.c_void_p]
    size = 1 << 20
    bufs = [ctypes.c_void_p(), ctypes.c_void_p()]
    for b in bufs:
        assert hip.hipHostMalloc(ctypes.byref(b), size, 0) == 0
    try:
        dst, src = bufs[0].value, bufs[1].value
        wl = W.custom([(64, 128)], n_shards=1, device="cpu")
        tab = wt.task_table(wl)
        tab.arr[0].shard_mem = wt.WT_MEM_PINNED_HOST
        tab.arr[0].shards[0].ptr = src
        wt.wt_plan_destroy(wt.wt_plan_create(tab, dst, wl.dst_bytes, wt.WT_MEM_PINNED_HOST))
        with pytest.raises(wt.WtError) as e:
            wt.wt_plan_create(tab, dst, size + 65536, wt.WT_MEM_PINNED_HOST)
        assert e.value.status == wt.WT_E_RANGE
        # 64 rows of 256 bytes starting 4 KiB before the end of the allocation
        tab.arr[0].shards[0].ptr = src + size - 4096
        with pytest.raises(wt.WtError) as e:
            wt.wt_plan_create(tab, dst, wl.dst_bytes, wt.WT_MEM_PINNED_HOST)
        assert e.value.status == wt.WT_E_RANGE
    finally:
        for b in bufs:
            hip.hipHostFree(b)