"""Seeded random plans against the oracle, bit for bit (marked gpu).

Each draw mixes what the other tests take one at a time: FP8 and BF16
outputs, fusion groups of 1-3 components, shapes that are tile multiples,
multiples of 8 or ragged, 1-9 shards (some empty), device or pinned-host
shards, a device or pinned-host destination, zero-copy or staged writes,
small watermarks and chunks (ring reuse), destination alignments of 2, 16
or 256 bytes, and both load hints. The whole destination region (canary
fill included) is compared with the oracle's image."""
import os
import random

import pytest
import torch

from bf16_fp8_weight_amd import workloads as W
from gpu_util import assert_images_equal, log, oracle_image_threaded, run_library

pytestmark = pytest.mark.gpu

COLS = [1, 3, 8, 24, 120, 128, 136, 256, 300, 384, 640, 1000, 1024, 2048]


def _draw(seed):
    rng = random.Random(seed)
    outs = []
    for i in range(rng.randint(1, 10)):
        kind = W.FP8 if rng.random() < 0.75 else W.BF16
        cols = rng.choice(COLS)
        n_parts = rng.choice([1, 1, 1, 2, 3])
        n_shards = rng.randint(1, 9)
        rows = [rng.choice([1, 7, 64, 128, 129, 200, 256, 384]) if rng.random() < 0.5 else rng.randint(1, 400)
                for _ in range(n_parts)]
        parts = W._matrix_parts([f"p{k}" for k in range(n_parts)], rows, n_shards)
        outs.append(W.OutputSpec(f"o{i}", kind, cols, parts))
    host = rng.random() < 0.4
    wl = W.Workload(f"random_{seed}", outs, seed=5000 + seed, shard_mem="host" if host else "device")
    wl.dst_bytes = W.pack(outs, align=rng.choice([2, 16, 256]))
    dist = rng.choice(["normal", "t"])
    gen = W._normal_bf16 if dist == "normal" else W._student_t3_bf16
    W._materialize(wl, "cuda", lambda o, p, g, d: gen((p.rows, o.cols), g, d))
    return wl, rng


def _seeds():
    # WT_RANDOM_PLAN_SEEDS=lo:hi runs seeds lo..hi-1 instead of the default 48
    spec = os.environ.get("WT_RANDOM_PLAN_SEEDS", "")
    if spec:
        lo, hi = (int(v) for v in spec.split(":"))
        return range(lo, hi)
    return range(48)


@pytest.mark.parametrize("seed", _seeds())
def test_random_plan(seed):
    from bf16_fp8_weight_amd import wt

    wl, rng = _draw(seed)
    dst_kind = wt.WT_MEM_PINNED_HOST if rng.random() < 0.3 else wt.WT_MEM_DEVICE
    o = wt.wt_plan_options_init()
    o.dst_write_mode = wt.WT_DST_STAGED if rng.random() < 0.3 else wt.WT_DST_ZERO_COPY
    o.chunk_bytes = rng.choice([0, 64 << 10, 1 << 20])
    o.load_hint = rng.choice([wt.WT_LOAD_AUTO, wt.WT_LOAD_PLAIN, wt.WT_LOAD_STREAM])
    o.watermark_bytes = 256 << 10
    tab = wt.task_table(wl)
    while True:  # smallest power-of-two watermark from 256 KiB that fits every output
        try:
            info = wt.wt_plan_check(tab, wl.dst_bytes, dst_kind, o)
            break
        except wt.WtError as e:
            assert e.status == wt.WT_E_WATERMARK, str(e)
            o.watermark_bytes *= 2
    log(f"  seed {seed}: {len(wl.outputs)} outputs, {wl.shard_mem} shards, dst {dst_kind}, mode {o.dst_write_mode}, "
        f"watermark {o.watermark_bytes >> 10} KiB, chunks {info['n_chunks']}, launches {info['n_launches']}")
    got, _ = run_library(wl, dst_kind=dst_kind, opts=o, table=tab)
    assert_images_equal(got, oracle_image_threaded(wl), wl)


def _replay_seeds():
    # WT_RANDOM_REPLAY_SEEDS=lo:hi runs seeds lo..hi-1 instead of the default 16
    spec = os.environ.get("WT_RANDOM_REPLAY_SEEDS", "")
    if spec:
        lo, hi = (int(v) for v in spec.split(":"))
        return range(lo, hi)
    return range(10000, 10016)


@pytest.mark.parametrize("seed", _replay_seeds())
def test_random_plan_replays(seed):
    # the same draws, replayed three times back to back with a random replay
    # depth and tile grouping; before the second and third replay every shard
    # is negated (device shards by a kernel on the replay stream, host shards
    # by the host after a synchronisation), so two negations bring the inputs
    # back to those the last replay read: the final image is the oracle's
    from bf16_fp8_weight_amd import wt

    wl, rng = _draw(seed)
    dst_kind = wt.WT_MEM_PINNED_HOST if rng.random() < 0.3 else wt.WT_MEM_DEVICE
    o = wt.wt_plan_options_init()
    o.dst_write_mode = wt.WT_DST_STAGED if rng.random() < 0.3 else wt.WT_DST_ZERO_COPY
    o.chunk_bytes = rng.choice([0, 64 << 10, 1 << 20])
    o.max_replays_in_flight = rng.choice([0, 1, 2, 3])
    o.tile_group = rng.choice([wt.WT_GROUP_AUTO, wt.WT_GROUP_SINGLE, wt.WT_GROUP_PAIR])
    o.watermark_bytes = 256 << 10
    tab = wt.task_table(wl)
    while True:
        try:
            wt.wt_plan_check(tab, wl.dst_bytes, dst_kind, o)
            break
        except wt.WtError as e:
            assert e.status == wt.WT_E_WATERMARK, str(e)
            o.watermark_bytes *= 2
    if dst_kind == wt.WT_MEM_DEVICE:
        dst = torch.full((wl.dst_bytes,), 0xA5, dtype=torch.uint8, device="cuda")
    else:
        dst = torch.full((wl.dst_bytes,), 0xA5, dtype=torch.uint8).pin_memory()
    h = wt.wt_plan_create(tab, dst.data_ptr(), wl.dst_bytes, dst_kind, o)
    host = wl.shard_mem == "host"
    try:
        s = torch.cuda.current_stream()
        for r in range(3):
            if r:
                if host:
                    s.synchronize()
                for out in wl.outputs:
                    for part in out.parts:
                        for sh in part.shards:
                            sh.neg_()
            wt.wt_prepare(h, s.cuda_stream)
        s.synchronize()
    finally:
        wt.wt_plan_destroy(h)
    log(f"  seed {seed}: {len(wl.outputs)} outputs, {wl.shard_mem} shards, depth {o.max_replays_in_flight}, "
        f"group {o.tile_group}, mode {o.dst_write_mode}")
    assert_images_equal(dst.cpu().numpy(), oracle_image_threaded(wl), wl)
