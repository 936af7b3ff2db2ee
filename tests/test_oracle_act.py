"""Pins of the oracle's block-scaled activation quantization
(oracle_quantize_act_b128): hand-worked blocks, reduction to the weight
path on one-row tensors, power-of-two scales against torch's cast, gather
and stride semantics. CPU only."""
import numpy as np
import pytest
import torch

import oracle
from golden_io import act_blocks


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _rand_bf16(rng, shape, std=0.02):
    return _bf16(rng.standard_normal(shape).astype(np.float32) * std)


@pytest.mark.parametrize("row", act_blocks(), ids=lambda r: r["name"])
def test_worked_blocks(row):
    q, s = oracle.quantize_act(row["x"][None, :])
    want = np.zeros(row["cols"], dtype=np.uint8)
    for c, b in row["bytes"].items():
        want[c] = b
    np.testing.assert_array_equal(q[0], want)
    assert [int(v) for v in s[0].view(np.uint32)] == row["scale_bits"]


@pytest.mark.parametrize("cols", [1, 8, 127, 128, 129, 300, 7168])
def test_row_equals_one_row_weight_tensor(cols):
    # a 1 x C tensor's 128 x 128 tiles are exactly its 1 x 128 blocks
    rng = np.random.default_rng(cols)
    x = _rand_bf16(rng, (5, cols))
    x[2, : min(cols, 128)] = 0  # a zero block
    q, s = oracle.quantize_act(x)
    nb = -(-cols // 128)
    for i in range(5):
        out = oracle.Output(kind=oracle.FP8_TILE128, cols=cols, parts=[[x[i:i + 1]]], dst_offset=0,
                            scale_offset=-(-cols // 16) * 16)
        img = oracle.prepare([out], out.scale_offset + 4 * nb)
        np.testing.assert_array_equal(q[i], img[:cols])
        np.testing.assert_array_equal(s[i].view(np.uint8), img[out.scale_offset:out.scale_offset + 4 * nb])


@pytest.mark.parametrize("k", [-20, -7, 0, 3])
def test_power_of_two_blocks_reduce_to_plain_cast(k):
    # amax = 448 * 2^k in every block => s = 2^k exactly and bytes = cast(x * 2^-k)
    rng = np.random.default_rng(100 + k)
    cols = 384
    v = rng.uniform(-448, 448, size=(3, cols)).astype(np.float32)
    v[:, ::128] = 448.0
    v = torch.from_numpy(v).to(torch.bfloat16).float().numpy()  # exactly representable values
    x = _bf16(v * np.float32(2.0 ** k))
    q, s = oracle.quantize_act(x)
    assert np.all(s == np.float32(2.0 ** k))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(q, ref)


def test_gather_and_strides():
    rng = np.random.default_rng(7)
    n_rows, cols, stride = 6, 200, 208
    x = _rand_bf16(rng, (n_rows, stride))
    idx = np.array([3, 0, 3, -1, 6, 5, 2**31 - 1], dtype=np.int32)
    q = np.full((idx.size, 224), 0xA5, dtype=np.uint8)
    sc = np.full((idx.size, 12), 0xA5, dtype=np.uint8)
    oracle.quantize_act(x, cols=cols, index=idx, q=q, scales=sc)
    dense_q, dense_s = oracle.quantize_act(np.ascontiguousarray(x[:, :cols]))
    for i, src in enumerate(idx):
        if 0 <= src < n_rows:
            np.testing.assert_array_equal(q[i, :cols], dense_q[src])
            np.testing.assert_array_equal(sc[i, :8], dense_s[src].view(np.uint8))
        else:
            assert np.all(q[i] == 0xA5) and np.all(sc[i] == 0xA5)
    assert np.all(q[:, cols:] == 0xA5) and np.all(sc[:, 8:] == 0xA5)


def test_rejects_bad_arguments():
    x = np.zeros((2, 128), dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.quantize_act(x, q=np.zeros((2, 100), dtype=np.uint8))          # q row shorter than cols
    with pytest.raises(ValueError):
        oracle.quantize_act(x, scales=np.zeros((2, 2), dtype=np.uint8))       # scale row shorter than one scale
    with pytest.raises(ValueError):
        oracle.quantize_act(x, cols=129)                                       # cols past the row stride
