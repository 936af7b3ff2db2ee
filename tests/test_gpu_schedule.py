"""The static schedule end to end on the GPU: metadata -> wt_schedule_build ->
one plan per source GPU (each prepares only the tensors assigned to it, into
the shared destination region) -> the region matches the oracle bit for bit.
On one GPU the sources run one after another. Marked gpu."""
import pytest
import torch

from bf16_fp8_weight_amd import workloads as W
from gpu_util import assert_images_equal, log, oracle_image_threaded

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("make,n_sources", [
    (lambda: W.dense_layer_h1024(device="cuda"), 2),
    (lambda: W.ragged_stress(device="cuda", n_tensors=24, max_dim=1000), 3),
    (lambda: W.mla_many_small(device="cuda", layers=1, n_small=200, host=True), 4),
])
def test_schedule_per_source_plans_compose(make, n_sources):
    from bf16_fp8_weight_amd import wt

    wl = make()
    log(f"  schedule {wl.name}: {len(wl.outputs)} outputs over {n_sources} sources")
    params, dsts = W.metadata(wl)
    sch = wt.Schedule(params, dsts, align=256, n_sources=n_sources)
    info = sch.info()
    assert info["dst_bytes"] == wl.dst_bytes
    dst = torch.full((wl.dst_bytes,), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream()
    used = 0
    for src in range(n_sources):
        tab = sch.tasks(src)
        if tab.n == 0:
            continue
        used += 1
        h = wt.wt_plan_create(tab, dst.data_ptr(), wl.dst_bytes, wt.WT_MEM_DEVICE)
        try:
            wt.wt_prepare(h, s.cuda_stream)
            s.synchronize()
        finally:
            wt.wt_plan_destroy(h)
    assert used >= 2
    assert_images_equal(dst.cpu().numpy(), oracle_image_threaded(wl), wl)


def test_source_plans_concurrently_on_separate_streams():
    # one plan per source, all replayed at once on their own streams into the
    # shared region (disjoint ranges): the result equals the oracle's image
    from bf16_fp8_weight_amd import wt

    wl = W.kimi_k2_expert_share(device="cuda", experts=6)
    params, dsts = W.metadata(wl)
    n_src = 3
    sch = wt.Schedule(params, dsts, align=256, n_sources=n_src)
    dst = torch.full((wl.dst_bytes,), 0xA5, dtype=torch.uint8, device="cuda")
    tabs = [sch.tasks(s) for s in range(n_src)]
    plans = [wt.wt_plan_create(t, dst.data_ptr(), wl.dst_bytes, wt.WT_MEM_DEVICE) for t in tabs if t.n]
    streams = [torch.cuda.Stream() for _ in plans]
    torch.cuda.synchronize()
    try:
        for _ in range(3):
            for h, s in zip(plans, streams):
                wt.wt_prepare(h, s.cuda_stream)
        for s in streams:
            s.synchronize()
    finally:
        for h in plans:
            wt.wt_plan_destroy(h)
    assert len(plans) == n_src
    assert_images_equal(dst.cpu().numpy(), oracle_image_threaded(wl), wl)
