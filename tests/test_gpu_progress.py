"""Completion counters on the GPU: the words a replay writes, what the host
may read once it sees one, replay numbering, and argument errors. Marked gpu."""
import ctypes

import numpy as np
import pytest
import torch

from bf16_fp8_weight_amd import workloads as W
from gpu_util import log, oracle_image_threaded

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wt():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)
    from bf16_fp8_weight_amd import wt as _wt
    yield _wt
    torch.cuda.synchronize()


def _words(n):
    return torch.zeros(n, dtype=torch.int64).pin_memory()


def _first_task_of_outputs(wl):
    firsts, t = [], 0
    for o in wl.outputs:
        firsts.append(t)
        t += len(o.parts)
    return firsts


def test_direct_launch_counts_replays(wt):
    wl = W.dense_layer_h1024(device="cuda")
    dst = torch.zeros(wl.dst_bytes, dtype=torch.uint8, device="cuda")
    plan = wt.Plan(wl, dst)
    assert plan.info()["n_units"] == 1
    w = _words(1)
    wt.wt_plan_set_progress(plan.handle, w.data_ptr(), 1)
    s = torch.cuda.current_stream()
    for r in range(1, 4):
        plan.prepare(s.cuda_stream)
        assert wt.wt_progress_wait(w.data_ptr(), r, 20 * 10**9)
    s.synchronize()
    assert int(w[0]) == 3
    assert not wt.wt_progress_wait(w.data_ptr(), 4, 10**6)  # nothing in flight: times out on the host
    # attaching again restarts the numbering; the words are left as they are
    wt.wt_plan_set_progress(plan.handle, w.data_ptr(), 1)
    w.zero_()
    plan.prepare(s.cuda_stream)
    s.synchronize()
    assert int(w[0]) == 1
    # detached: no more writes
    wt.wt_plan_set_progress(plan.handle, 0, 0)
    plan.prepare(s.cuda_stream)
    s.synchronize()
    assert int(w[0]) == 1
    np.testing.assert_array_equal(dst.cpu().numpy(), oracle_image_threaded(wl, fill=0))
    plan.close()


@pytest.mark.parametrize("mode", ["zero_copy", "staged"])
def test_pipeline_units_readable_when_seen(wt, mode):
    # pinned-host shards and a pinned-host destination: the host reads each
    # unit's bytes straight from the region as soon as its word turns 1,
    # while later units are still in flight
    wl = W.mla_many_small(device="cuda", layers=1, n_small=300, host=True)
    dst = torch.full((wl.dst_bytes,), 0xA5, dtype=torch.uint8).pin_memory()
    o = wt.wt_plan_options_init()
    o.watermark_bytes = 160 << 20 if mode == "zero_copy" else 256 << 20
    o.chunk_bytes = 8 << 20
    o.dst_write_mode = wt.WT_DST_STAGED if mode == "staged" else wt.WT_DST_ZERO_COPY
    plan = wt.Plan(wl, dst, wt.WT_MEM_PINNED_HOST, o)
    n = plan.info()["n_units"]
    log(f"  {wl.name} {mode}: {n} completion units")
    assert n >= 3
    firsts = _first_task_of_outputs(wl)
    unit_of = [wt.wt_plan_task_unit(plan.handle, t) for t in firsts]
    assert sorted(set(unit_of)) == list(range(n)) and unit_of == sorted(unit_of)
    with pytest.raises(wt.WtError):
        wt.wt_plan_task_unit(plan.handle, sum(len(x.parts) for x in wl.outputs))
    w = _words(n)
    wt.wt_plan_set_progress(plan.handle, w.data_ptr(), n)
    want = oracle_image_threaded(wl)
    view = dst.numpy()
    s = torch.cuda.current_stream()
    plan.prepare(s.cuda_stream)
    snaps = []
    for u in range(n):
        assert wt.wt_progress_wait(w.data_ptr() + 8 * u, 1, 60 * 10**9), f"unit {u} not reached"
        outs = [i for i, x in enumerate(unit_of) if x == u]
        snaps.append((outs, [view[r0:r1].copy() for r0, r1 in _ranges(wl, outs)]))
    s.synchronize()
    assert w.tolist() == [1] * n
    for outs, got in snaps:
        for (r0, r1), g in zip(_ranges(wl, outs), got):
            assert np.array_equal(g, want[r0:r1]), f"bytes [{r0}, {r1}) not final when their unit was seen"
    assert np.array_equal(view, want)
    plan.close()


def _ranges(wl, outs):
    r = []
    for i in outs:
        o = wl.outputs[i]
        r.append((o.dst_offset, o.dst_offset + o.data_bytes))
        if o.kind == W.FP8:
            r.append((o.scale_offset, o.scale_offset + o.scale_bytes))
    return r


def test_set_progress_rejects_bad_words(wt):
    wl = W.custom([(256, 256)], n_shards=2, device="cuda")
    dst = torch.zeros(wl.dst_bytes, dtype=torch.uint8, device="cuda")
    plan = wt.Plan(wl, dst)
    w = _words(4)
    dev = torch.zeros(4, dtype=torch.int64, device="cuda")
    host = np.zeros(4, dtype=np.int64)  # pageable
    for ptr, n in [(w.data_ptr(), 0), (w.data_ptr() + 4, 1), (dev.data_ptr(), 1), (host.ctypes.data, 1)]:
        with pytest.raises(wt.WtError) as e:
            wt.wt_plan_set_progress(plan.handle, ptr, n)
        assert e.value.status == wt.WT_E_INVAL
    wt.wt_plan_set_progress(plan.handle, w.data_ptr(), 4)
    plan.close()
