"""The oracle's pins catch plausible mistakes (CPU only).

Each case copies oracle.c to a temporary directory, plants one mistake by a
textual replacement, builds it with gcc and runs the CPU pin suite against
that library (WT_ORACLE_LIB). Every mutant must make at least one pin fail.
The real oracle source is never modified.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("ties_away_from_zero", "if (rest > half || (rest == half && (code & 1u))) code += 1u;",
     "if (rest >= half) code += 1u;"),
    ("truncate_instead_of_round", "if (rest > half || (rest == half && (code & 1u))) code += 1u;", ";"),
    ("subnormal_ties_away", "if (rest > half || (rest == half && (k & 1u))) k += 1u;", "if (rest >= half) k += 1u;"),
    ("subnormal_shift_off_by_one", "const int shift = 14 - e;", "const int shift = 15 - e;"),
    ("no_saturation", "if (mag >= 0x43E00000u) return sign | 0x7Eu;", "if (mag >= 0x7F800000u) return sign | 0x7Eu;"),
    ("nan_to_max", "if (mag > 0x7F800000u) return sign | 0x7Fu;", "if (mag > 0x7F800000u) return sign | 0x7Eu;"),
    ("sign_dropped_on_underflow", "if (e < -17) return sign;", "if (e < -17) return 0;"),
    ("wrong_exponent_bias", "uint32_t code = ((uint32_t)(e + 7) << 3) | (frac >> 20);",
     "uint32_t code = ((uint32_t)(e + 8) << 3) | (frac >> 20);"),
    ("reciprocal_multiply", "const float q = x / s;", "const float q = x * (1.0f / s);"),
    ("multiply_by_scale", "const float q = x / s;", "const float q = x * s;"),
    ("scale_uses_447", "return amax / 448.0f;", "return amax / 447.0f;"),
    ("zero_tile_scale_448", "if (amax == 0.0f) return 1.0f;", "if (amax == 0.0f) return 1.0f / 448.0f;"),
    ("scale_grid_transposed", "memcpy(scales + 4 * (I * tiles_c + J), &s, sizeof s);",
     "memcpy(scales + 4 * (J * tiles_r + I), &s, sizeof s);"),
    ("amax_without_abs", "const float a = fabsf(oracle_bf16_to_f32(x[r * C + c]));",
     "const float a = oracle_bf16_to_f32(x[r * C + c]);"),
    ("amax_skips_last_row", "for (int64_t r = r0; r < r1; ++r)\n        for (int64_t c = c0; c < c1; ++c) {",
     "for (int64_t r = r0; r < r1 - 1; ++r)\n        for (int64_t c = c0; c < c1; ++c) {"),
    ("shards_reversed", "const oracle_shard *sh = &part->shards[k];\n      if (sh->rows > 0)",
     "const oracle_shard *sh = &part->shards[part->n_shards - 1 - k];\n      if (sh->rows > 0)"),
    ("components_overwrite", "fused_row += Rc;", "fused_row += 0;"),
    ("tile_rows_127", "const int64_t r0 = 128 * I, r1 = (128 * I + 128 < R) ? 128 * I + 128 : R;",
     "const int64_t r0 = 128 * I, r1 = (128 * I + 127 < R) ? 128 * I + 127 : R;"),
    # fp32 pattern ranges (the reference of the exhaustive cast check)
    ("range_offset_by_one", "const uint32_t bits = first + (uint32_t)i;",
     "const uint32_t bits = first + (uint32_t)i + 1u;"),
    ("range_saturates_instead_of_wrapping", "const uint32_t bits = first + (uint32_t)i;",
     "const uint32_t bits = (uint64_t)first + i > 0xFFFFFFFFull ? 0xFFFFFFFFu : first + (uint32_t)i;"),
    # block-scaled activations
    ("act_block_127", "const int64_t c0 = 128 * b, c1 = (c0 + 128 < cols) ? c0 + 128 : cols;",
     "const int64_t c0 = 128 * b, c1 = (c0 + 127 < cols) ? c0 + 127 : cols;"),
    ("act_index_ignored", "const int64_t src = index ? (int64_t)index[i] : i;", "const int64_t src = i < n_rows ? i : 0;"),
    ("act_scales_packed", "memcpy(scales + i * s_stride + 4 * b, &s, sizeof s);",
     "memcpy(scales + i * 4 * nb + 4 * b, &s, sizeof s);"),
    ("act_amax_signed", "const float a = fabsf(oracle_bf16_to_f32(xr[c]));", "const float a = oracle_bf16_to_f32(xr[c]);"),
    ("act_q_dense_rows", "q[i * q_stride + c] = oracle_quantize_element(xr[c], s);",
     "q[i * cols + c] = oracle_quantize_element(xr[c], s);"),
]

PIN_FILES = ["tests/test_oracle_cast.py", "tests/test_oracle_quant.py", "tests/test_oracle_prepare.py",
             "tests/test_oracle_act.py"]


def _run_mutant(name, old, new, tmp):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    d = os.path.join(tmp, name)
    os.makedirs(d)
    open(os.path.join(d, "oracle.c"), "w").write(src.replace(old, new))
    open(os.path.join(d, "oracle.h"), "w").write(open(os.path.join(ROOT, "oracle", "oracle.h")).read())
    so = os.path.join(d, "liboracle.so")
    subprocess.run(["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
                    os.path.join(d, "oracle.c"), "-o", so, "-lm"], check=True)
    env = dict(os.environ, WT_ORACLE_LIB=so, WT_SLOW="0")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PIN_FILES],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode, r.stdout[-2000:]


def test_every_planted_mistake_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda m: _run_mutant(*m, tmp), MUTANTS))
    survivors = [(n, out) for n, rc, out in results if rc == 0]
    assert not survivors, "mutants not caught by any pin: " + ", ".join(n for n, _ in survivors)
    # a crash is not a catch: each mutant must fail an assertion (rc 1)
    crashed = [(n, rc) for n, rc, _ in results if rc not in (0, 1)]
    assert not crashed, crashed
