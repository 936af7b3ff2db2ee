"""The plain-C program tests/c_abi/c_gpu_prepare (C99 + the HIP runtime +
libwt.so, built by the repository's build step) drives the whole GPU path
through the C ABI with no Python in its process: shards in device memory,
wt_plan_create, wt_prepare replays, wt_plan_destroy. The destination image
it writes must equal the oracle's bit for bit. Marked gpu."""
import os
import struct
import subprocess

import numpy as np
import pytest
import torch

from bf16_fp8_weight_amd import workloads as W
from gpu_util import assert_images_equal, oracle_image_threaded

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "c_gpu_prepare")


def _write_input(wl, path):
    """Task table and shard bytes in the program's input format: one task per
    fusion component, components of a fused output sharing a fusion group."""
    head, data = [], []
    n_tasks = 0
    for oi, o in enumerate(wl.outputs):
        fused = len(o.parts) > 1
        for p in o.parts:
            n_tasks += 1
            dtype = 0 if o.kind == W.FP8 else 1
            head.append(struct.pack("<iiiiqQQ", len(p.shard_rows), dtype, oi if fused else -1, 0, o.cols,
                                    o.dst_offset, o.scale_offset))
            head.append(struct.pack(f"<{len(p.shard_rows)}q", *p.shard_rows))
            for s, r in zip(p.shards, p.shard_rows):
                if r:
                    data.append(s.detach().cpu().contiguous().view(torch.int16).numpy().tobytes())
    with open(path, "wb") as f:
        f.write(b"WTC1" + struct.pack("<IQ", n_tasks, wl.dst_bytes))
        for h in head:
            f.write(h)
        for d in data:
            f.write(d)


@pytest.mark.parametrize("make", [
    lambda: W.dense_layer_h1024(device="cpu"),
    lambda: W.custom([(300, 1000), (129, 17), (1, 300), (256, 640)], n_shards=3, device="cpu", seed=41),
], ids=["dense_layer_h1024", "ragged_mix"])
def test_c_program_matches_oracle(tmp_path, make):
    assert os.path.exists(EXE), "tests/c_abi/c_gpu_prepare is not built (run the build step)"
    wl = make()
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    _write_input(wl, inp)
    r = subprocess.run([EXE, str(inp), str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "c gpu prepare ok" in r.stdout, r.stdout + r.stderr
    got = np.fromfile(out, dtype=np.uint8)
    assert got.size == wl.dst_bytes
    assert_images_equal(got, oracle_image_threaded(wl), wl)


def test_c_program_back_to_back_replays(tmp_path):
    # 2,000 replays of the one-layer plan issued back to back from C: the
    # image is still the oracle's, and the time per replay on the stream and
    # per call on the host is reported (the library's replay cost without
    # Python or timing events between the calls)
    assert os.path.exists(EXE), "tests/c_abi/c_gpu_prepare is not built (run the build step)"
    wl = W.dense_layer_h1024(device="cpu")
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    _write_input(wl, inp)
    r = subprocess.run([EXE, str(inp), str(out), "2001"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "c gpu prepare ok" in r.stdout, r.stdout + r.stderr
    print(r.stdout.strip(), flush=True)
    assert "2000 replays back to back" in r.stdout
    got = np.fromfile(out, dtype=np.uint8)
    assert_images_equal(got, oracle_image_threaded(wl), wl)
