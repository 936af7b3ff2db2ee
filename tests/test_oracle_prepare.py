"""Pins of the oracle's assembly, fusion, tiling and packing (CPU only).

Pins: pass-through output equals torch.cat of the shard bytes; FP8 output of
a fused tensor whose components are multiples of 128 rows equals the
concatenation of the components quantized alone; the result does not depend
on the shard split (even, uneven, empty shards) or on task order; tiny and
ragged shapes against a numpy/torch tile loop whose cast is torch's; bytes
outside the output ranges are never written; invariants of every tile of the
dense hidden-1024 layer.
"""
import numpy as np
import pytest
import torch

import brute
import oracle_glue
from bf16_fp8_weight_amd import workloads as W
from oracle import BF16_COPY, FP8_TILE128, Output


def _bits(shape, seed, dist="normal"):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g) * 0.02
    if dist == "t":
        x = x / torch.sqrt((torch.randn(shape, generator=g) ** 2 + torch.randn(shape, generator=g) ** 2) / 2)
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _split(x, n):
    rows = W.split_rows(x.shape[0], n)
    out, r = [], 0
    for k in rows:
        out.append(x[r:r + k])
        r += k
    return out


def _library_reference(x_bits):
    """Tile loop with numpy amax, numpy fp32 division and torch's E4M3 cast
    (valid because every quotient of a tile is below 464 in magnitude)."""
    R, C = x_bits.shape
    x = brute.bf16_bits_to_f32(x_bits)
    q = np.zeros((R, C), dtype=np.uint8)
    tr, tc = -(-R // 128), -(-C // 128)
    sc = np.zeros((tr, tc), dtype=np.float32)
    for I in range(tr):
        for J in range(tc):
            blk = x[128 * I:128 * I + 128, 128 * J:128 * J + 128]
            a = np.float32(np.abs(blk).max())
            s = np.float32(1.0) if a == 0 else a / np.float32(448.0)
            sc[I, J] = s
            q[128 * I:128 * I + 128, 128 * J:128 * J + 128] = (
                torch.from_numpy(np.ascontiguousarray(blk / s)).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    return q, sc


def _run(oracle_lib, outs, nbytes, fill=0):
    return oracle_lib.prepare(outs, nbytes, np.full(nbytes, fill, dtype=np.uint8))


@pytest.mark.parametrize("shape", [(1, 1), (1, 129), (129, 1), (128, 128), (129, 129), (3000, 1), (257, 300), (5, 1000)])
def test_tiny_and_ragged_shapes(oracle_lib, shape):
    x = _bits(shape, seed=sum(shape), dist="t")
    R, C = shape
    tiles = (-(-R // 128)) * (-(-C // 128))
    so = R * C + (-(R * C)) % 4
    img = _run(oracle_lib, [Output(FP8_TILE128, C, [_split(x, 3)], 0, so)], so + 4 * tiles)
    q, sc = _library_reference(x)
    assert np.array_equal(img[:R * C].reshape(R, C), q)
    assert np.array_equal(img[so:].view(np.float32).reshape(sc.shape), sc)


def test_passthrough_is_concatenation(oracle_lib):
    a, b = _bits((37, 5), 1), _bits((64, 5), 2)
    o = Output(BF16_COPY, 5, [_split(a, 4), _split(b, 8)], dst_offset=16)
    img = _run(oracle_lib, [o], 16 + 2 * 101 * 5 + 16, fill=0xA5)
    want = torch.cat([torch.from_numpy(a.view(np.int16)), torch.from_numpy(b.view(np.int16))]).numpy().view(np.uint8).ravel()
    assert np.array_equal(img[16:16 + want.size], want)
    assert np.all(img[:16] == 0xA5) and np.all(img[16 + want.size:] == 0xA5)


def test_fused_equals_concat_of_separate(oracle_lib):
    C = 384
    a, b, c = _bits((256, C), 3), _bits((128, C), 4), _bits((384, C), 5)
    ta = lambda r: (-(-r // 128)) * 3
    n_q = (256 + 128 + 384) * C
    fused = Output(FP8_TILE128, C, [_split(a, 2), _split(b, 3), _split(c, 8)], 0, n_q)
    img_f = _run(oracle_lib, [fused], n_q + 4 * ta(768))
    sep, off, soff, imgs = [], 0, 0, []
    for x in (a, b, c):
        R = x.shape[0]
        img = _run(oracle_lib, [Output(FP8_TILE128, C, [[x]], 0, R * C)], R * C + 4 * ta(R))
        imgs.append(img)
    want_q = np.concatenate([im[:x.shape[0] * C] for im, x in zip(imgs, (a, b, c))])
    want_s = np.concatenate([im[x.shape[0] * C:] for im, x in zip(imgs, (a, b, c))])
    assert np.array_equal(img_f[:n_q], want_q)
    assert np.array_equal(img_f[n_q:], want_s)


def test_fusion_tiles_straddle_components(oracle_lib):
    # components of 100 and 90 rows: tile row 0 mixes both; the fused-tensor
    # rule (quantize the concatenation) decides, checked by the library loop
    C = 200
    a, b = _bits((100, C), 6), _bits((90, C), 7)
    R = 190
    so = R * C
    img = _run(oracle_lib, [Output(FP8_TILE128, C, [_split(a, 3), _split(b, 2)], 0, so)], so + 4 * 4)
    q, sc = _library_reference(np.concatenate([a, b]))
    assert np.array_equal(img[:so].reshape(R, C), q)
    assert np.array_equal(img[so:].view(np.float32).reshape(2, 2), sc)


@pytest.mark.parametrize("n", [1, 2, 3, 7, 8, 64, 300])
def test_result_independent_of_shard_split(oracle_lib, n):
    x = _bits((300, 256), 8)
    so = 300 * 256
    ref = _run(oracle_lib, [Output(FP8_TILE128, 256, [[x]], 0, so)], so + 4 * 6)
    img = _run(oracle_lib, [Output(FP8_TILE128, 256, [_split(x, n)], 0, so)], so + 4 * 6)
    assert np.array_equal(img, ref)


def test_shard_order_matters(oracle_lib):
    # assembling in rank order is part of the definition: swapping two shards
    # changes the result (guards against an order-insensitive assembly)
    x = _bits((256, 128), 9)
    sh = _split(x, 2)
    so = 256 * 128
    a = _run(oracle_lib, [Output(FP8_TILE128, 128, [sh], 0, so)], so + 8)
    b = _run(oracle_lib, [Output(FP8_TILE128, 128, [sh[::-1]], 0, so)], so + 8)
    assert not np.array_equal(a, b)
    assert np.array_equal(a[:128 * 128], b[128 * 128:so]) and np.array_equal(a[so:so + 4], b[so + 4:so + 8])


def test_task_order_and_canary(oracle_lib):
    wl = W.custom([(200, 160), (64, 64), (1, 300), (129, 17)], n_shards=3, seed=11)
    outs = oracle_glue.oracle_outputs(wl)
    ref = oracle_lib.prepare(outs, wl.dst_bytes, np.full(wl.dst_bytes, 0x5A, dtype=np.uint8))
    perm = [2, 0, 3, 1]
    img = oracle_lib.prepare([outs[i] for i in perm], wl.dst_bytes, np.full(wl.dst_bytes, 0x5A, dtype=np.uint8))
    assert np.array_equal(img, ref)
    # every byte outside the data and scale ranges still holds the canary
    mask = np.zeros(wl.dst_bytes, dtype=bool)
    for o in wl.outputs:
        mask[o.dst_offset:o.dst_offset + o.data_bytes] = True
        mask[o.scale_offset:o.scale_offset + o.scale_bytes] = True
    assert np.all(ref[~mask] == 0x5A)


def test_range_errors(oracle_lib):
    x = _bits((4, 4), 1)
    with pytest.raises(ValueError):
        oracle_lib.prepare([Output(FP8_TILE128, 4, [[x]], 10, 0)], 16)  # data runs past the end
    with pytest.raises(ValueError):
        oracle_lib.prepare([Output(FP8_TILE128, 4, [[x]], 0, 14)], 16)  # scale runs past the end
    with pytest.raises(ValueError):
        oracle_lib.prepare([Output(BF16_COPY, 4, [[x]], 1, 0)], 32)


def test_dense_layer_invariants(oracle_lib):
    wl = W.dense_layer_h1024()
    img = oracle_glue.oracle_image(wl)
    for o in wl.outputs:
        R, C = o.rows, o.cols
        x = np.concatenate([oracle_glue.full_bits(p, C) for p in o.parts])
        xf = brute.bf16_bits_to_f32(x)
        q = img[o.dst_offset:o.dst_offset + R * C].reshape(R, C)
        s = img[o.scale_offset:o.scale_offset + o.scale_bytes].view(np.float32).reshape(R // 128, C // 128)
        for I in range(R // 128):
            for J in range(C // 128):
                blk = xf[128 * I:128 * I + 128, 128 * J:128 * J + 128]
                qb = q[128 * I:128 * I + 128, 128 * J:128 * J + 128]
                a = np.abs(blk).max()
                assert s[I, J] == a / np.float32(448.0)
                # amax -> +-448
                at = np.abs(blk) == a
                assert np.all((qb[at] & 0x7F) == 0x7E)
                # x-space half-ulp bound with the stored scale (slack for the quotient rounding)
                v = brute.e4m3_value(qb)
                E = (qb >> 3) & 0xF
                ulp = np.where(E == 0, 2.0 ** -9, np.exp2(E.astype(np.float64) - 10))
                err = np.abs(v * np.float64(s[I, J]) - blk.astype(np.float64))
                assert np.all(err <= ulp / 2 * np.float64(s[I, J]) * (1 + 2.0 ** -18))
                # sign preserved
                assert np.all((qb >> 7) == (np.signbit(blk)).astype(np.uint8))
