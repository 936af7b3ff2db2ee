"""Pins of the oracle's tile scale and per-element quantization (CPU only).

Definition pinned: s = amax / 448 in fp32 (1 for an all-zero tile), and each
element becomes cast(fl32(x / s)). Pins: hand-worked tiles (tests/golden),
numpy's IEEE fp32 division for every BF16 amax, torch's x / s followed by
torch's float8_e4m3fn cast over (x, amax) pairs, the exact power-of-two scale
case, amax -> +-448 for every BF16 amax, and the half-ulp error bound.
"""
import numpy as np
import pytest
import torch

import brute
import golden_io
from oracle import BF16_COPY, FP8_TILE128, Output

# every positive finite BF16 value (the possible non-zero tile amax values)
POS_BF16 = np.arange(1, 0x7F80, dtype=np.uint16)


def test_worked_tiles(oracle_lib):
    for t in golden_io.worked_tiles():
        bits = golden_io.f32_to_bf16_bits_exact(t["x"])
        R, C = t["rows"], t["cols"]
        o = Output(FP8_TILE128, C, [[bits]], dst_offset=0, scale_offset=R * C + (-(R * C) % 4))
        n = o.scale_offset + 4
        img = oracle_lib.prepare([o], n)
        assert np.array_equal(img[:R * C].reshape(R, C), t["bytes"]), t["name"]
        s_bits = int(img[o.scale_offset:o.scale_offset + 4].view(np.uint32)[0])
        assert s_bits == t["scale_bits"], (t["name"], hex(s_bits))


def test_scale_for_every_bf16_amax(oracle_lib):
    amax = brute.bf16_bits_to_f32(POS_BF16)
    want = amax / np.float32(448.0)  # numpy fp32 IEEE division
    got = np.array([oracle_lib.tile_scale(float(a)) for a in amax], dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert oracle_lib.tile_scale(0.0) == 1.0
    # distinct amax give distinct scales; 1,247 of them are fp32-subnormal
    assert np.unique(got).size == got.size
    assert int(np.sum(got < np.finfo(np.float32).tiny)) == 1247


def test_amax_maps_to_448_for_every_bf16_amax(oracle_lib):
    # the element equal to the tile amax always lands on +-448 (0x7E / 0xFE)
    amax = brute.bf16_bits_to_f32(POS_BF16)
    s = np.array([oracle_lib.tile_scale(float(a)) for a in amax], dtype=np.float32)
    q = amax / s
    assert q.min() >= 447.0 and q.max() < 449.0
    pos = np.array([oracle_lib.quantize_elements(np.array([b], np.uint16), float(si))[0]
                    for b, si in zip(POS_BF16[::37], s[::37])])
    assert np.all(pos == 0x7E)
    neg = np.array([oracle_lib.quantize_elements(np.array([b | 0x8000], np.uint16), float(si))[0]
                    for b, si in zip(POS_BF16[::37], s[::37])])
    assert np.all(neg == 0xFE)


def _domain_check(oracle_lib, amax_bits):
    xb = np.arange(65536, dtype=np.uint32)
    x = brute.bf16_bits_to_f32(xb)
    got = oracle_lib.quantize_domain(amax_bits)
    for i, ab in enumerate(amax_bits):
        a = brute.bf16_bits_to_f32(np.array([ab]))[0]
        inside = np.isfinite(x) & (np.abs(x) <= a)
        s = torch.tensor([a], dtype=torch.float32)
        s = torch.where(s == 0, torch.ones_like(s), s / 448.0)
        q = torch.from_numpy(x[inside]) / s  # torch fp32 IEEE division
        want = q.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        row = got[i][inside]
        bad = np.nonzero(row != want)[0]
        assert bad.size == 0, (hex(int(ab)), [(float(x[inside][j]), hex(row[j]), hex(want[j])) for j in bad[:5]])


def test_quantize_domain_vs_torch_sampled(oracle_lib):
    # a stride through all positive BF16 amax, every subnormal-scale amax near
    # the fp32 subnormal boundary, the power-of-two scales, and amax = 0
    pick = set(POS_BF16[::61].tolist())
    pick |= set(range(0x0001, 0x0010)) | set(range(0x0370, 0x0380)) | set(range(0x3F00, 0x3F08))
    pick |= {int(golden_io.f32_to_bf16_bits_exact(np.float32(448.0 * 2.0 ** k))) for k in range(-40, 1)}
    pick.add(0)
    _domain_check(oracle_lib, np.array(sorted(pick), dtype=np.uint16))


@pytest.mark.slow
def test_quantize_domain_vs_torch_exhaustive(oracle_lib):
    amax = np.concatenate([[0], POS_BF16]).astype(np.uint16)
    for a in range(0, amax.size, 512):
        _domain_check(oracle_lib, amax[a:a + 512])


def test_power_of_two_scale_reduces_to_plain_cast(oracle_lib):
    # amax = 448 * 2^k gives s = 2^k exactly, so q = x * 2^-k exactly and the
    # bytes equal torch's cast of x * 2^-k
    xb = np.arange(65536, dtype=np.uint32)
    x = brute.bf16_bits_to_f32(xb)
    for k in [-20, -7, -1, 0, 3, 10]:
        s = oracle_lib.tile_scale(448.0 * 2.0 ** k)
        assert s == 2.0 ** k
        inside = np.isfinite(x) & (np.abs(x) <= 448.0 * 2.0 ** k)
        got = oracle_lib.quantize_elements(xb[inside].astype(np.uint16), s)
        want = torch.from_numpy(x[inside] * np.float32(2.0 ** -k)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(got, want), k


def test_half_ulp_bound(oracle_lib):
    # |val(byte) - fl(x/s)| <= ulp/2 in quotient space (equality only at ties,
    # which must land on an even code); ulp = 2^(E-10) for normal codes and
    # 2^-9 for subnormal codes
    rng = np.random.default_rng(5)
    for amax in [1e-30, 1e-6, 0.02, 0.5, 3.0, 448.0, 3e4]:
        a = np.float32(amax)
        xs = (rng.uniform(-1, 1, 200000) * a).astype(np.float32)
        xb = (xs.view(np.uint32) >> 16).astype(np.uint16)  # truncation to BF16: any BF16 values will do
        x = brute.bf16_bits_to_f32(xb)
        amax_eff = np.abs(x).max()
        s = np.float32(oracle_lib.tile_scale(float(amax_eff)))
        q = (x / s).astype(np.float64)
        b = oracle_lib.quantize_elements(xb, float(s))
        v = brute.e4m3_value(b)
        E = (b >> 3) & 0xF
        ulp = np.where(E == 0, 2.0 ** -9, np.exp2(E.astype(np.float64) - 10))
        err = np.abs(v - q)
        assert np.all(err <= ulp / 2), amax
        tie = err == ulp / 2
        assert np.all((b[tie] & 1) == 0)


def test_zero_tile(oracle_lib):
    x = np.zeros((128, 128), dtype=np.uint16)
    x[::3, ::5] = 0x8000  # -0.0
    o = Output(FP8_TILE128, 128, [[x]], dst_offset=0, scale_offset=128 * 128)
    img = oracle_lib.prepare([o], 128 * 128 + 4)
    assert img[128 * 128:].view(np.float32)[0] == 1.0
    assert np.array_equal(img[:128 * 128].reshape(128, 128), np.where(x == 0x8000, 0x80, 0).astype(np.uint8))
