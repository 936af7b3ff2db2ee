"""Block-scaled (1 x 128) FP8 quantization of token activations on the GPU
(wt_quantize_act_b128 through the C ABI) against the oracle, bit for bit:
the MoE dispatch sender shape (128 tokens x 7168, top-8 gather into
interleaved send-buffer slots), a 4096-token batch, ragged shapes and
strides, unaligned addresses (general path), out-of-range and repeated
indices, every finite BF16 magnitude, pinned-host outputs. Marked gpu."""
import os

import numpy as np
import pytest
import torch

import oracle
from bf16_fp8_weight_amd import workloads as W
from gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wt():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)
    from bf16_fp8_weight_amd import wt as _wt
    yield _wt
    torch.cuda.synchronize()


def _u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _run(wt, x, cols, x_stride, index, n_out, q, q_stride, sc, s_stride, x_off=0, n_rows=None):
    """x: device BF16 storage (flat); q/sc: uint8 tensors (device or pinned)."""
    n_rows = x.numel() // x_stride if n_rows is None else n_rows
    s = torch.cuda.current_stream()
    wt.wt_quantize_act_b128(x.data_ptr() + 2 * x_off, n_rows, cols, x_stride,
                            index.data_ptr() if index is not None else 0, n_out,
                            q.data_ptr(), q_stride, sc.data_ptr(), s_stride, s.cuda_stream)
    s.synchronize()


def _oracle(x_u16, cols, index, n_out, q_stride, s_stride):
    q = np.full((n_out, q_stride), 0xA5, dtype=np.uint8)
    sc = np.full((n_out, s_stride), 0xA5, dtype=np.uint8)
    idx = None if index is None else index.cpu().numpy()
    oracle.quantize_act(x_u16, cols=cols, index=idx, n_out=n_out, q=q, scales=sc)
    return q, sc


def _check_separate(wt, x2d, cols, index=None, n_out=None, q_stride=None, s_stride=None, host_out=False):
    n_rows, x_stride = x2d.shape
    n_out = (n_rows if index is None else index.numel()) if n_out is None else n_out
    nb = -(-cols // 128)
    q_stride = cols if q_stride is None else q_stride
    s_stride = 4 * nb if s_stride is None else s_stride
    mk = (lambda n: torch.full((n,), 0xA5, dtype=torch.uint8).pin_memory()) if host_out else \
        (lambda n: torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda"))
    q = mk(max(1, n_out * q_stride))
    sc = mk(max(1, n_out * s_stride))
    _run(wt, x2d.reshape(-1), cols, x_stride, index, n_out, q, q_stride, sc, s_stride)
    wq, ws = _oracle(_u16(x2d), cols, index, n_out, q_stride, s_stride)
    gq = q.cpu().numpy()[: n_out * q_stride].reshape(n_out, q_stride)
    gs = sc.cpu().numpy()[: n_out * s_stride].reshape(n_out, s_stride)
    bad = np.argwhere(gq != wq)
    assert bad.size == 0, f"{bad.shape[0]} code bytes differ, first at (row, col) {tuple(bad[0])}"
    bad = np.argwhere(gs != ws)
    assert bad.size == 0, f"{bad.shape[0]} scale bytes differ, first at (row, byte) {tuple(bad[0])}"


def test_dispatch_decode_interleaved_slots(wt):
    wl = W.act_dispatch(device="cuda")
    log(f"  {wl.name}: {wl.n_out} rows, slot {wl.slot} B")
    H, nb, slot = wl.hidden, wl.nb, wl.slot
    buf = torch.full((wl.n_out * slot,), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream()
    wt.wt_quantize_act_b128(wl.x.data_ptr(), wl.tokens, H, H, wl.index.data_ptr(), wl.n_out,
                            buf.data_ptr(), slot, buf.data_ptr() + H, slot, s.cuda_stream)
    s.synchronize()
    wq, ws = _oracle(_u16(wl.x), H, wl.index, wl.n_out, H, 4 * nb)
    want = np.full((wl.n_out, slot), 0xA5, dtype=np.uint8)
    want[:, :H] = wq
    want[:, H:H + 4 * nb] = ws
    got = buf.cpu().numpy().reshape(wl.n_out, slot)
    assert np.array_equal(got, want)


def test_token_batch_4096(wt):
    wl = W.act_tokens(device="cuda", tokens=4096)
    _check_separate(wt, wl.x, wl.hidden)


@pytest.mark.parametrize("cols,x_pad,q_pad,s_pad", [
    (1, 0, 0, 0), (7, 5, 3, 4), (8, 0, 0, 0), (127, 1, 1, 0), (128, 8, 8, 4), (129, 3, 0, 8),
    (300, 4, 4, 0), (1003, 1, 7, 12), (7168, 0, 16, 0), (4096 + 8, 8, 0, 4),
])
def test_ragged_shapes_and_strides(wt, cols, x_pad, q_pad, s_pad):
    g = torch.Generator(device="cuda")
    g.manual_seed(cols)
    n_rows = 37
    x = W._activations((n_rows, cols + x_pad), g, "cuda")
    _check_separate(wt, x, cols, q_stride=cols + q_pad, s_stride=4 * (-(-cols // 128)) + s_pad)


def test_gather_repeats_and_out_of_range(wt):
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    x = W._activations((50, 1024), g, "cuda")
    idx = torch.tensor([3, 3, 49, 0, -1, 50, 2**31 - 1, -(2**31), 7, 7, 7], dtype=torch.int32, device="cuda")
    _check_separate(wt, x, 1024, index=idx)
    # without an index, output rows past n_rows are skipped
    _check_separate(wt, x, 1024, n_out=53)


def test_general_path_unaligned(wt):
    # x shifted by one element (2 bytes) and q by one byte: not 16/8-aligned
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    n_rows, cols = 19, 520
    base = W._activations((1, n_rows * cols + 1), g, "cuda").reshape(-1)
    q = torch.full((n_rows * cols + 1,), 0xA5, dtype=torch.uint8, device="cuda")
    sc = torch.full((n_rows * 20,), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream()
    wt.wt_quantize_act_b128(base.data_ptr() + 2, n_rows, cols, cols, 0, n_rows, q.data_ptr() + 1, cols,
                            sc.data_ptr(), 20, s.cuda_stream)
    s.synchronize()
    x2d = base[1:].reshape(n_rows, cols)
    wq, ws = _oracle(_u16(x2d), cols, None, n_rows, cols, 20)
    gq = q.cpu().numpy()
    assert gq[0] == 0xA5
    assert np.array_equal(gq[1:].reshape(n_rows, cols), wq)
    assert np.array_equal(sc.cpu().numpy().reshape(n_rows, 20), ws)


def test_every_finite_bf16_magnitude(wt):
    # random finite BF16 bit patterns: block amax from subnormal to 3.4e38,
    # so both division forms and every exponent of the cast are exercised
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 1 << 16, size=(512, 2048), dtype=np.uint32).astype(np.uint16)
    expo = (bits >> 7) & 0xFF
    bits[expo == 0xFF] &= 0x807F  # NaN / inf -> a subnormal of the same sign
    # scale each block's range: shift exponents down by a per-block amount
    blocks = bits.reshape(512, 16, 128)
    shift = rng.integers(0, 250, size=(512, 16, 1)).astype(np.int32)
    e = ((blocks >> 7) & 0xFF).astype(np.int32)
    e2 = np.clip(e - shift, 0, 254)
    blocks = ((blocks & 0x807F) | (e2.astype(np.uint16) << 7)).astype(np.uint16)
    x = torch.from_numpy(blocks.reshape(512, 2048).view(np.int16)).cuda().view(torch.bfloat16)
    _check_separate(wt, x, 2048)


def test_pinned_host_outputs(wt):
    g = torch.Generator(device="cuda")
    g.manual_seed(13)
    x = W._activations((64, 7168), g, "cuda")
    _check_separate(wt, x, 7168, host_out=True)


def test_argument_errors(wt):
    x = torch.zeros((4, 256), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros(4 * 256, dtype=torch.uint8, device="cuda")
    sc = torch.zeros(64, dtype=torch.uint8, device="cuda")

    def st(**kw):
        a = dict(x=x.data_ptr(), n_rows=4, cols=256, x_row_stride=256, row_index=0, n_out=4, q=q.data_ptr(),
                 q_row_stride=256, scales=sc.data_ptr(), scale_row_stride=8, stream=0)
        a.update(kw)
        try:
            wt.wt_quantize_act_b128(**a)
            return 0
        except wt.WtError as e:
            return e.status
    assert st() == 0
    torch.cuda.synchronize()
    assert st(n_rows=-1) == wt.WT_E_INVAL
    assert st(cols=0) == wt.WT_E_INVAL
    assert st(x_row_stride=255) == wt.WT_E_INVAL
    assert st(q_row_stride=200) == wt.WT_E_INVAL
    assert st(scale_row_stride=4) == wt.WT_E_INVAL
    assert st(q=0) == wt.WT_E_INVAL
    assert st(x=x.data_ptr() + 1) == wt.WT_E_ALIGN
    assert st(scales=sc.data_ptr() + 2) == wt.WT_E_ALIGN
    assert st(n_out=0, q=0, scales=0) == 0  # no-op


def _seeds():
    # WT_RANDOM_ACT_SEEDS=lo:hi runs seeds lo..hi-1 instead of the default 24
    spec = os.environ.get("WT_RANDOM_ACT_SEEDS", "")
    if spec:
        lo, hi = (int(v) for v in spec.split(":"))
        return range(lo, hi)
    return range(24)


@pytest.mark.parametrize("seed", _seeds())
def test_random_shapes_strides_and_gathers(wt, seed):
    import random
    rng = random.Random(seed)
    cols = rng.choice([1, 5, 8, 64, 127, 128, 200, 1024, 1031, 7168])
    n_rows = rng.randint(1, 300)
    x_stride = cols + rng.choice([0, 0, 1, 8, 13])
    nb = -(-cols // 128)
    q_stride = cols + rng.choice([0, 0, 3, 8, 64])
    s_stride = 4 * nb + rng.choice([0, 0, 4, 12])
    if rng.random() < 0.5:
        n_out = rng.randint(0, 400)
        idx = torch.tensor([rng.randint(-3, n_rows + 2) for _ in range(n_out)], dtype=torch.int32, device="cuda")
    else:
        idx, n_out = None, rng.randint(0, n_rows + 3)
    g = torch.Generator(device="cuda")
    g.manual_seed(900 + seed)
    x_off = rng.choice([0, 0, 1])  # one element: breaks 16-byte alignment (general path)
    base = W._activations((1, n_rows * x_stride + x_off), g, "cuda").reshape(-1)
    host_out = rng.random() < 0.25
    mk = (lambda n: torch.full((n,), 0xA5, dtype=torch.uint8).pin_memory()) if host_out else \
        (lambda n: torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda"))
    q = mk(max(1, n_out * q_stride))
    sc = mk(max(1, n_out * s_stride))
    s = torch.cuda.current_stream()
    wt.wt_quantize_act_b128(base.data_ptr() + 2 * x_off, n_rows, cols, x_stride,
                            idx.data_ptr() if idx is not None else 0, n_out, q.data_ptr(), q_stride,
                            sc.data_ptr(), s_stride, s.cuda_stream)
    s.synchronize()
    x2d = base[x_off:].reshape(n_rows, x_stride)
    wq, ws = _oracle(_u16(x2d), cols, idx, n_out, q_stride, s_stride)
    gq = q.cpu().numpy()[: n_out * q_stride].reshape(n_out, q_stride)
    gs = sc.cpu().numpy()[: n_out * s_stride].reshape(n_out, s_stride)
    assert np.array_equal(gq, wq) and np.array_equal(gs, ws), \
        f"seed {seed}: rows {n_rows} cols {cols} strides {x_stride}/{q_stride}/{s_stride} n_out {n_out}"
