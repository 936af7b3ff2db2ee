"""bench.py's command line on the CPU: asked for several GPUs it refuses with
a message and exit code 2 before touching a GPU (the path runs on one)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)
    assert not r.stdout.strip().startswith("{")  # no result line


def test_verification_leg_on_the_cpu():
    # the bench's oracle leg on a tiny workload: an image equal to the
    # oracle's verifies, one changed byte does not; the baseline record names
    # its threads, the CPU and a single-threaded rate
    import importlib.util

    import numpy as np
    import torch

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle_glue
    from bf16_fp8_weight_amd import workloads as W

    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    wl = W.custom([(200, 136), (64, 72)], n_shards=3, device="cpu")
    img = oracle_glue.oracle_image(wl, fill=0xA5)
    cpu, ok = bench._verify(wl, torch.from_numpy(img.copy()), threads=2)
    assert ok is True
    for k in ("value", "cores", "threads", "cpu_model", "machine_cores", "single_thread_GBps", "all_cores_GBps"):
        assert k in cpu, k
    assert cpu["cores"] == cpu["threads"] == 2 and cpu["kind"] == "oracle"
    bad = img.copy()
    bad[wl.outputs[1].dst_offset + 5] ^= 1
    _, ok = bench._verify(wl, torch.from_numpy(bad), threads=2, baseline=False)
    assert ok is False
    assert bench._shards_per_tensor(wl) == 3
