"""Parity of the HIP path (through the C ABI) with the CPU oracle, bit for
bit, on the five workloads and on edge cases. Marked gpu."""
import numpy as np
import pytest
import torch

from bf16_fp8_weight_amd import workloads as W
from gpu_util import Timer, assert_images_equal, log, oracle_image_threaded, run_library

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from bf16_fp8_weight_amd import wt  # noqa: F401  (fails loudly if libwt.so is missing)
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _parity(wl, **kw):
    log(f"  workload {wl.name}: {len(wl.outputs)} outputs, {wl.input_bytes / 1e6:.1f} MB in, seed {wl.seed}")
    with Timer("gpu"):
        got, info = run_library(wl, **kw)
    with Timer("oracle"):
        want = oracle_image_threaded(wl)
    assert_images_equal(got, want, wl)
    return info


def test_dense_layer_h1024():
    wl = W.dense_layer_h1024(device="cuda")
    info = _parity(wl)
    assert info["n_launches"] == 1


@pytest.mark.parametrize("hint", [1, 2])
def test_load_hints_same_bytes(hint):
    from bf16_fp8_weight_amd import wt

    wl = W.custom([(512, 2048), (384, 7168), (256, 4096)], n_shards=2, device="cuda")
    o = wt.wt_plan_options_init()
    o.load_hint = hint
    _parity(wl, opts=o)


@pytest.mark.parametrize("hint", [1, 2])
def test_tile_groups_with_leftovers(hint):
    # rows of 3 and 5 full tiles: pairs plus a single tile at the end of each band;
    # 1 and 2 full tiles; a band split across shards (edge tiles) next to paired bands
    from bf16_fp8_weight_amd import wt

    wl = W.custom([(384, 384), (256, 640), (128, 128), (256, 256), (512, 1152)], n_shards=4, device="cuda",
                  dist="t")
    o = wt.wt_plan_options_init()
    o.load_hint = hint
    o.tile_group = wt.WT_GROUP_PAIR  # a small plan: pairs only when asked for
    _parity(wl, opts=o)


def test_plan_context_manager():
    # the binding's Plan destroys its plan when the with-block ends
    from bf16_fp8_weight_amd import wt

    wl = W.custom([(256, 384)], n_shards=2, device="cuda", seed=36)
    dst = torch.full((wl.dst_bytes,), 0xA5, dtype=torch.uint8, device="cuda")
    with wt.Plan(wl, dst) as plan:
        plan.prepare(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
    assert plan.handle == 0
    assert_images_equal(dst.cpu().numpy(), oracle_image_threaded(wl), wl)


def test_ragged_stress_reduced():
    wl = W.ragged_stress(device="cuda", n_tensors=40, max_dim=1400)
    _parity(wl)


@pytest.mark.parametrize("shapes,n_shards,align", [
    ([(1, 1), (1, 129), (129, 1), (128, 128), (129, 129), (3000, 1)], 3, 256),
    ([(1, 8), (8, 8), (127, 136), (300, 264), (1000, 24)], 8, 256),   # aligned fast path, tiny/edge tiles
    ([(200, 160), (64, 64), (129, 17)], 300, 256),                    # many empty shards
    ([(257, 512), (100, 4096)], 1, 1),                                 # unaligned destination offsets
])
def test_edge_shapes(shapes, n_shards, align):
    wl = W.custom(shapes, n_shards=n_shards, device="cuda", align=align, dist="t")
    _parity(wl)


def test_fused_components_straddling_tiles():
    wl = W.custom([(100, 256), (90, 256), (200, 256)], n_shards=3, device="cuda", fused=True)
    _parity(wl)


def test_single_row_shards():
    wl = W.custom([(130, 1024)], n_shards=130, device="cuda", fused=False)
    _parity(wl)


def test_task_order_independent():
    from bf16_fp8_weight_amd import wt
    wl = W.custom([(300, 512), (64, 64), (1, 300), (129, 17), (256, 1024)], n_shards=3, device="cuda")
    ref, _ = run_library(wl)
    tab = wt.task_table(wl)
    tasks = [tab.arr[i] for i in range(tab.n)]
    perm = [3, 0, 4, 2, 1]
    shuffled = wt.TaskTable([])
    arr = (wt.wt_task * len(perm))()
    for j, i in enumerate(perm):
        arr[j] = tasks[i]
    shuffled.arr, shuffled.n, shuffled._shards = arr, len(perm), tab._shards
    got, _ = run_library(wl, table=shuffled)
    assert np.array_equal(got, ref)


def test_new_contents_same_plan():
    # the plan fixes addresses; contents change every step
    from bf16_fp8_weight_amd import wt
    wl = W.custom([(384, 1024), (256, 256)], n_shards=4, device="cuda")
    dst = torch.full((wl.dst_bytes,), 0xA5, dtype=torch.uint8, device="cuda")
    tab = wt.task_table(wl)
    h = wt.wt_plan_create(tab, dst.data_ptr(), wl.dst_bytes)
    try:
        for step in range(3):
            g = torch.Generator(device="cuda").manual_seed(100 + step)
            for o in wl.outputs:
                for p in o.parts:
                    for s in p.shards:
                        s.copy_((torch.randn(s.shape, generator=g, device="cuda") * (0.01 * (step + 1))).to(torch.bfloat16))
            wt.wt_prepare(h, torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            want = oracle_image_threaded(wl)
            assert_images_equal(dst.cpu().numpy(), want, wl)
    finally:
        wt.wt_plan_destroy(h)


def test_consumers_on_the_replay_stream_see_the_bytes():
    # work enqueued on the replay's stream right behind it sees the new bytes
    # with only that stream synchronized: a device-to-host copy into pinned
    # memory and a device-side clone, while the contents change every step
    from bf16_fp8_weight_amd import wt
    wl = W.custom([(384, 1024), (256, 256), (129, 40)], n_shards=4, device="cuda")
    dst = torch.full((wl.dst_bytes,), 0xA5, dtype=torch.uint8, device="cuda")
    host = torch.empty(wl.dst_bytes, dtype=torch.uint8, pin_memory=True)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    h = wt.wt_plan_create(wt.task_table(wl), dst.data_ptr(), wl.dst_bytes)
    try:
        for step in range(4):
            g = torch.Generator(device="cuda").manual_seed(200 + step)
            with torch.cuda.stream(s):
                for o in wl.outputs:
                    for p in o.parts:
                        for sh in p.shards:
                            sh.copy_((torch.randn(sh.shape, generator=g, device="cuda") * (0.02 * (step + 1)))
                                     .to(torch.bfloat16))
                wt.wt_prepare(h, s.cuda_stream)
                host.copy_(dst, non_blocking=True)
                clone = dst.clone()
            s.synchronize()
            want = oracle_image_threaded(wl)
            assert_images_equal(host.numpy(), want, wl)
            assert_images_equal(clone.cpu().numpy(), want, wl)
    finally:
        wt.wt_plan_destroy(h)


@pytest.mark.parametrize("host", [False, True])
def test_destroy_right_after_prepare(host):
    # destroy waits for the plan's enqueued work (the launch on the caller's
    # stream, or the pipeline streams) before freeing its tables and staging
    from bf16_fp8_weight_amd import wt
    if host:
        wl = W.mla_many_small(device="cuda", layers=1, n_small=100, host=True)
    else:
        wl = W.custom([(4096, 2048), (2048, 4096)], n_shards=4, device="cuda")
    dst = torch.full((wl.dst_bytes,), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    h = wt.wt_plan_create(wt.task_table(wl), dst.data_ptr(), wl.dst_bytes)
    wt.wt_prepare(h, s.cuda_stream)
    wt.wt_plan_destroy(h)
    s.synchronize()
    assert_images_equal(dst.cpu().numpy(), oracle_image_threaded(wl), wl)


def test_dense_7b_full():
    wl = W.dense_7b(device="cuda")
    _parity(wl)


def test_kimi_k2_moe_full():
    wl = W.kimi_k2_expert_share(device="cuda")
    _parity(wl)


def test_ragged_stress_full():
    wl = W.ragged_stress(device="cuda")
    _parity(wl)


def _scaled_workload(shapes, scales, seed, n_shards=2):
    """custom() workload whose tensors are multiplied by per-tensor scales (in
    fp32, then rounded to BF16) to reach extreme magnitudes."""
    wl = W.custom(shapes, n_shards=n_shards, device="cuda", seed=seed)
    for o, sc in zip(wl.outputs, scales):
        for p in o.parts:
            for sh in p.shards:
                sh.copy_((sh.to(torch.float32) * sc).to(torch.bfloat16))
    return wl


def test_extreme_magnitudes():
    # tiny tiles take the kernel's IEEE-division branch (s < 2^-100), BF16
    # subnormals included; huge tiles approach the BF16 maximum
    shapes = [(256, 256), (128, 384), (300, 136), (130, 1000), (256, 128)]
    scales = [1e-30, 1e-36, 3e-39, 1e34, 1e-25]
    _parity(_scaled_workload(shapes, scales, seed=31))


def test_extreme_magnitudes_general_path():
    # the same magnitudes on odd row lengths: full and partial general tiles
    # through the IEEE-division branch (s < 2^-100), BF16 subnormals included
    shapes = [(256, 385), (128, 129), (300, 257), (130, 1001), (256, 127)]
    scales = [1e-30, 1e-36, 3e-39, 1e34, 1e-25]
    _parity(_scaled_workload(shapes, scales, seed=35))


def test_row_wider_than_fast_path_limit():
    # 2^24 + 8 columns: beyond the aligned path's 32-bit tile offsets, so the
    # general path takes it
    _parity(W.custom([(2, (1 << 24) + 8)], n_shards=2, device="cuda", seed=32))


@pytest.mark.parametrize("C", [(1 << 24) - 1, (1 << 24) + 1])
def test_general_full_tiles_at_the_offset_limit(C):
    # 128 x C with C odd, so the general path. Below 2^24 its full tiles store
    # through 32-bit offsets that reach 127 C + 127, just under 2^31; above,
    # they take 64-bit addresses. The whole output would keep the oracle busy
    # for minutes, so tile columns are checked one by one: a tile depends on
    # its own 128 x 128 values only, so a 128-column slice of the input,
    # prepared alone, gives the same bytes.
    import oracle

    wl = W.custom([(128, C)], n_shards=2, device="cuda", seed=34)
    got, info = run_library(wl)
    tiles_c = -(-C // 128)
    assert info["n_general_tiles"] == tiles_c
    o = wl.outputs[0]
    x = torch.cat(list(o.parts[0].shards), dim=0)
    data = got[o.dst_offset:o.dst_offset + 128 * C].reshape(128, C)
    for J in (0, 1, tiles_c // 2, tiles_c - 2, tiles_c - 1):
        c0 = 128 * J
        w = min(128, C - c0)
        bits = x[:, c0:c0 + w].contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
        want = oracle.prepare([oracle.Output(oracle.FP8_TILE128, w, [[bits]], 0, 128 * w)], 128 * w + 4,
                              np.zeros(128 * w + 4, dtype=np.uint8))
        assert np.array_equal(data[:, c0:c0 + w], want[:128 * w].reshape(128, w)), f"tile column {J}"
        assert bytes(got[o.scale_offset + 4 * J:o.scale_offset + 4 * J + 4]) == bytes(want[128 * w:]), f"scale {J}"


def test_single_large_tensor():
    # one 2 GiB tensor (2^30 elements) in 8 shards
    _parity(W.custom([(65536, 16384)], n_shards=8, device="cuda", seed=33))
