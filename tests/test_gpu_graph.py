"""Graph capture of the library's launches (marked gpu): a device-resident
plan with completion words, and the activation quantization, captured into a
HIP graph (through torch.cuda.graph) and replayed several times with eager
work and synchronisations in between; every replay is checked against the
oracle (new shard contents each time) and the completion word against the
number of replays. Pipelined plans refuse capture (WT_E_STATE)."""
import numpy as np
import pytest
import torch

import oracle
from bf16_fp8_weight_amd import workloads as W
from gpu_util import assert_images_equal, oracle_image_threaded

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wt():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)
    from bf16_fp8_weight_amd import wt as _wt
    yield _wt
    torch.cuda.synchronize()


def _refill(wl, step):
    g = torch.Generator(device="cuda").manual_seed(700 + step)
    for o in wl.outputs:
        for p in o.parts:
            for s in p.shards:
                s.copy_((torch.randn(s.shape, generator=g, device="cuda") * 0.01 * (step + 1)).to(torch.bfloat16))


def test_captured_plan_with_completion_words(wt):
    wl = W.custom([(512, 1024), (384, 2048), (130, 136)], n_shards=3, device="cuda")
    dst = torch.full((wl.dst_bytes,), 0xA5, dtype=torch.uint8, device="cuda")
    plan = wt.Plan(wl, dst)
    words = torch.zeros(1, dtype=torch.int64).pin_memory()
    wt.wt_plan_set_progress(plan.handle, words.data_ptr(), 1)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up outside capture
        plan.prepare(side.cuda_stream)
    side.synchronize()
    assert int(words[0]) == 1
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.prepare(torch.cuda.current_stream().cuda_stream)
    for step in range(4):
        _refill(wl, step)                        # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert_images_equal(dst.cpu().numpy(), oracle_image_threaded(wl), wl)
        # the replay counter lives in device memory, so each replay of the graph advances it
        assert int(words[0]) == 2 + step
    plan.prepare(torch.cuda.current_stream().cuda_stream)  # eager replay after the graph ones
    torch.cuda.synchronize()
    assert int(words[0]) == 6
    del graph
    plan.close()


def test_captured_activation_quantization(wt):
    g = torch.Generator(device="cuda").manual_seed(31)
    x = W._activations((128, 7168), g, "cuda")
    idx = torch.randint(0, 128, (1024,), generator=g, device="cuda", dtype=torch.int32)
    q = torch.full((1024 * 7168,), 0xA5, dtype=torch.uint8, device="cuda")
    sc = torch.full((1024 * 224,), 0xA5, dtype=torch.uint8, device="cuda")

    def launch():
        wt.wt_quantize_act_b128(x.data_ptr(), 128, 7168, 7168, idx.data_ptr(), 1024, q.data_ptr(), 7168,
                                sc.data_ptr(), 224, torch.cuda.current_stream().cuda_stream)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch()
    side.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(8):  # eight launches per graph replay, as a dispatch loop would issue
            launch()
    for step in range(3):
        x.copy_(W._activations((128, 7168), g, "cuda"))   # eager work between replays
        q.fill_(0xA5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        xb = x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        wq = np.full((1024, 7168), 0xA5, dtype=np.uint8)
        ws = np.full((1024, 224), 0xA5, dtype=np.uint8)
        oracle.quantize_act(xb, cols=7168, index=idx.cpu().numpy(), n_out=1024, q=wq, scales=ws)
        assert np.array_equal(q.cpu().numpy().reshape(1024, 7168), wq)
        assert np.array_equal(sc.cpu().numpy().reshape(1024, 224), ws)
    del graph


def _refill_host(wl, step):
    g = torch.Generator().manual_seed(900 + step)
    for o in wl.outputs:
        for p in o.parts:
            for s in p.shards:
                if s.numel():
                    s.copy_((torch.randn(s.shape, generator=g) * 0.02 * (step + 1)).to(torch.bfloat16))


def test_pipelined_plan_refuses_capture(wt):
    wl = W.mla_many_small(device="cuda", layers=1, n_small=50, host=True)
    dst = torch.zeros(wl.dst_bytes, dtype=torch.uint8, device="cuda")
    plan = wt.Plan(wl, dst)
    assert plan.info()["n_chunks"] > 0
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(wt.WtError) as e:
        with torch.cuda.graph(graph):
            plan.prepare(torch.cuda.current_stream().cuda_stream)
    assert e.value.status == wt.WT_E_STATE
    torch.cuda.synchronize()
    plan.prepare(torch.cuda.current_stream().cuda_stream)  # still usable outside capture
    torch.cuda.synchronize()
    assert_images_equal(dst.cpu().numpy(), oracle_image_threaded(wl, fill=0), wl)
    plan.close()


@pytest.mark.skip(reason="capture of pipelined replays is withdrawn: a build that captured them (stage streams "
                         "forked from and joined to the caller's stream, no host-side waits) ended in a "
                         "segmentation fault inside the runtime's end of capture on MI355X, cause not found; "
                         "pipelined plans return WT_E_STATE under capture (test_pipelined_plan_refuses_capture)")
@pytest.mark.parametrize("mode", ["h2d_device_dst", "staged_host_dst"])
def test_captured_pipelined_plan(wt, mode):
    # shards in pinned host memory: the pipeline (host-to-device copies, one
    # launch per chunk, and in staged mode copies into a pinned-host region)
    # captured into a graph; new host contents before each replay, every
    # replay compared with the oracle, then an eager replay after the graph's
    wl = W.mla_many_small(device="cuda", layers=1, n_small=50, host=True)
    o = wt.wt_plan_options_init()
    # just above the largest output's staging (o: 117 MB of BF16 in, 176 MB
    # staged in and out), so the ring is reused within the replay
    o.watermark_bytes = 128 << 20
    o.chunk_bytes = 8 << 20
    if mode == "staged_host_dst":
        o.watermark_bytes = 192 << 20
        o.dst_write_mode = wt.WT_DST_STAGED
        dst = torch.full((wl.dst_bytes,), 0xA5, dtype=torch.uint8).pin_memory()
        kind = wt.WT_MEM_PINNED_HOST
    else:
        dst = torch.full((wl.dst_bytes,), 0xA5, dtype=torch.uint8, device="cuda")
        kind = wt.WT_MEM_DEVICE
    plan = wt.Plan(wl, dst, kind, o)
    assert plan.info()["n_chunks"] > 2
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up outside capture
        plan.prepare(side.cuda_stream)
    side.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.prepare(torch.cuda.current_stream().cuda_stream)
    for step in range(3):
        _refill_host(wl, step)                   # host work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert_images_equal(dst.cpu().numpy(), oracle_image_threaded(wl), wl)
    _refill_host(wl, 7)
    plan.prepare(torch.cuda.current_stream().cuda_stream)  # eager replay after the graph ones
    torch.cuda.synchronize()
    assert_images_equal(dst.cpu().numpy(), oracle_image_threaded(wl), wl)
    del graph
    plan.close()
