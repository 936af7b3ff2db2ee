"""Independent brute-force E4M3 helpers for pinning the oracle.

Nothing here is shared with the oracle or the GPU library. The grid of E4M3
values is enumerated from the OCP FP8 specification's E4M3 encoding (bias 7,
subnormals m * 2^-9, S.1111.111 reserved for NaN, no infinity); the nearest
grid point is then found by exhaustive distance comparison, which is a
different algorithm from the oracle's bit manipulation.
"""
import numpy as np


def e4m3_magnitudes():
    """(codes, values): the 127 non-negative finite E4M3 codes 0x00..0x7E and
    their exact values, enumerated from exponent/mantissa fields."""
    codes, vals = [], []
    for E in range(16):
        for m in range(8):
            if E == 15 and m == 7:
                continue  # NaN
            v = m * 2.0 ** -9 if E == 0 else (1.0 + m / 8.0) * 2.0 ** (E - 7)
            codes.append((E << 3) | m)
            vals.append(v)
    return np.array(codes, dtype=np.uint8), np.array(vals, dtype=np.float64)


CODES, VALS = e4m3_magnitudes()


def nearest_even_bruteforce(x):
    """E4M3 byte for float values x by exhaustive search over all 127 finite
    magnitudes: nearest value, ties to the even code, saturating; NaN ->
    S.1111.111. x is any float array (held exactly in float64)."""
    x = np.asarray(x, dtype=np.float64).ravel()
    out = np.empty(x.size, dtype=np.uint8)
    sign = np.signbit(x).astype(np.uint8) << 7
    mag = np.abs(x)
    nan = np.isnan(x)
    big = ~nan & (mag >= VALS[-1])
    rest = ~nan & ~big
    m = mag[rest]
    # distance to every grid value, chunked to bound memory
    res = np.empty(m.size, dtype=np.uint8)
    step = 1 << 15
    for a in range(0, m.size, step):
        d = np.abs(m[a:a + step, None] - VALS[None, :])
        dmin = d.min(axis=1, keepdims=True)
        cand = d == dmin
        # among the (one or two) nearest, prefer the even code
        even = (CODES[None, :] & 1) == 0
        two = cand.sum(axis=1) > 1
        pick = np.where(two[:, None], cand & even, cand)
        res[a:a + step] = CODES[np.argmax(pick, axis=1)]
    out[rest] = res
    out[big] = 0x7E
    out[nan] = 0x7F
    return out | sign


def midpoint_table_cast(x32):
    """E4M3 byte for fp32 values via a sorted midpoint table (searchsorted),
    ties resolved to the even code. Vectorised for large samples."""
    x = np.asarray(x32, dtype=np.float32).ravel()
    sign = (x.view(np.uint32) >> 24).astype(np.uint8) & 0x80
    mag = np.abs(x.astype(np.float64))
    mids = (VALS[1:] + VALS[:-1]) / 2.0
    idx = np.searchsorted(mids, mag, side="left")  # mag <= mids[idx]
    idx = np.minimum(idx, VALS.size - 1)
    # exactly on a midpoint: between idx and idx+1, take the even code
    on_mid = np.zeros(mag.size, dtype=bool)
    valid = idx < mids.size
    on_mid[valid] = mag[valid] == mids[idx[valid]]
    up = on_mid & ((CODES[np.minimum(idx, VALS.size - 1)] & 1) == 1)
    idx = np.where(up, idx + 1, idx)
    code = CODES[np.minimum(idx, VALS.size - 1)]
    code = np.where(mag >= VALS[-1], np.uint8(0x7E), code)
    code = np.where(np.isnan(mag), np.uint8(0x7F), code)
    return (code | sign).astype(np.uint8)


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def e4m3_value(byte):
    """Exact value of an E4M3 byte (float64), NaN for S.1111.111."""
    b = np.asarray(byte, dtype=np.uint8)
    E = (b >> 3) & 0xF
    m = (b & 7).astype(np.float64)
    v = np.where(E == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(E.astype(np.float64) - 7))
    v = np.where((E == 15) & ((b & 7) == 7), np.nan, v)
    return np.where(b & 0x80, -v, v)
