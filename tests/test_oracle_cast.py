"""Pins of the oracle's fp32 -> E4M3 cast (CPU only).

The cast is defined by the OCP FP8 E4M3 encoding with round to nearest, ties
to even, and saturation to +-448. It is pinned by: the specification's
characteristic values and hand-derived tie cases (tests/golden), exhaustive
brute-force nearest search over all 65,536 BF16 inputs, a midpoint-table cast
over a large fp32 sample, and torch's own float8_e4m3fn conversion as a third
implementation wherever torch's non-saturating conversion is defined the same
way (|q| < 464).
"""
import numpy as np
import pytest
import torch

import brute
import golden_io


def test_golden_e4m3_values(oracle_lib):
    for v, want in golden_io.e4m3_values():
        got = oracle_lib.cast_e4m3fn(np.array([v], dtype=np.float32))[0]
        assert got == want, f"cast({v!r}) = {got:#04x}, expected {want:#04x}"


def test_value_of_every_byte(oracle_lib):
    # the oracle's decoder agrees with the enumerated grid for every byte
    for b in range(256):
        got = oracle_lib.e4m3fn_value(b)
        want = float(brute.e4m3_value(np.uint8(b)))
        assert (np.isnan(got) and np.isnan(want)) or got == want, b


def test_cast_all_bf16_patterns_vs_bruteforce(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32)
    x = brute.bf16_bits_to_f32(bits)
    got = oracle_lib.cast_e4m3fn(x)
    want = brute.nearest_even_bruteforce(x)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(int(bits[i])), float(x[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


def _fp32_sample():
    # every fp32 pattern whose low 8 bits are one of a few values: covers
    # every exponent and the bit patterns around each E4M3 rounding boundary
    hi = np.arange(1 << 24, dtype=np.uint32) << 8
    return np.concatenate([hi, hi | 1, hi | 0x80, hi | 0xFF]).view(np.float32)


def test_cast_fp32_sample_vs_midpoint_table(oracle_lib):
    x = _fp32_sample()
    got = oracle_lib.cast_e4m3fn(x)
    want = brute.midpoint_table_cast(x)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(int(x.view(np.uint32)[i])), hex(got[i]), hex(want[i])) for i in bad[:10]]


def test_midpoint_table_agrees_with_bruteforce_near_boundaries():
    # the two independent test-side casts agree on every midpoint and its
    # fp32 neighbours, so the large-sample pin above rests on two methods
    mids = ((brute.VALS[1:] + brute.VALS[:-1]) / 2).astype(np.float32)
    u = mids.view(np.uint32)
    x = np.concatenate([u - 1, u, u + 1]).view(np.float32)
    x = np.concatenate([x, -x])
    assert np.array_equal(brute.midpoint_table_cast(x), brute.nearest_even_bruteforce(x))


def test_cast_vs_torch_float8(oracle_lib):
    x = _fp32_sample()
    finite = np.isfinite(x) & (np.abs(x) < 464.0)
    xs = x[finite]
    got = oracle_lib.cast_e4m3fn(xs)
    want = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(xs[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


@pytest.mark.slow
def test_cast_all_fp32_patterns_vs_midpoint_table(oracle_lib):
    step = 1 << 26
    for first in range(0, 1 << 32, step):
        got = oracle_lib.cast_f32_range(first, step)
        x = (np.arange(step, dtype=np.uint64) + first).astype(np.uint32).view(np.float32)
        want = brute.midpoint_table_cast(x)
        assert np.array_equal(got, want), hex(first)


def _range_bits(first, count):
    return ((np.arange(count, dtype=np.uint64) + np.uint64(first)) & np.uint64(0xFFFFFFFF)).astype(np.uint32)


def _range_windows():
    """(first, count) windows of consecutive fp32 patterns: zero and the
    subnormals above it, every E4M3 rounding boundary (the midpoints between
    adjacent E4M3 magnitudes) of both signs with its fp32 neighbours, the
    saturation threshold 448 and the first non-representable magnitudes
    above it, infinity and the NaNs past it (both signs), and a window that
    wraps past 0xFFFFFFFF back to 0."""
    w = [(0, 1 << 20), (0x80000000, 1 << 16), (0x3A000000, 1 << 22)]
    mids = ((brute.VALS[1:] + brute.VALS[:-1]) / 2).astype(np.float32).view(np.uint32)
    for m in mids:
        w.append((int(m) - 32, 64))
        w.append((int(m | 0x80000000) - 32, 64))
    for centre in (0x43E00000, 0x43E80000, 0x43F00000, 0x7F800000, 0xFF800000):
        w.append((centre - 4096, 8192))
    w.append((0xFFFFF000, 0x2000))
    return w


def test_cast_f32_range_windows_vs_midpoint_table(oracle_lib):
    # oracle_cast_f32_range walks consecutive fp32 patterns first + i
    # (modulo 2^32); checked window by window against the test-side
    # midpoint-table cast of the same patterns, and against brute-force
    # nearest search on the boundary windows
    for first, count in _range_windows():
        got = oracle_lib.cast_f32_range(first, count)
        x = _range_bits(first, count).view(np.float32)
        want = brute.midpoint_table_cast(x)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (hex(first), [(hex(int(x.view(np.uint32)[i])), hex(got[i]), hex(want[i]))
                                            for i in bad[:5]])
        if count <= 8192:
            assert np.array_equal(got, brute.nearest_even_bruteforce(x)), hex(first)


def test_cast_f32_range_wraps_modulo_2_32(oracle_lib):
    # the window crossing 0xFFFFFFFF ends with the largest-magnitude negative
    # NaN patterns (-> 0xFF) and continues at +0 (-> 0x00)
    got = oracle_lib.cast_f32_range(0xFFFFFFFE, 4)
    assert list(got) == [0xFF, 0xFF, 0x00, 0x00]
