/*
 * oracle.c -- plain, slow, single-threaded CPU reference for parameter
 * preparation. TEST INFRASTRUCTURE ONLY (see oracle.h for the definition and
 * the readings it follows). Written for a reader who checks it against the
 * definition by eye: assemble, fuse, then loop over tiles and elements, with
 * no blocking, fusion of loops or reordering.
 *
 * Build: gcc -std=c11 -O2 -fno-fast-math -ffp-contract=off -shared -fPIC
 * (no flush-to-zero: subnormal scales and inputs are part of the domain).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

float oracle_bf16_to_f32(uint16_t bits) {
  /* BF16 is the upper half of an fp32 pattern. */
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/*
 * E4M3 (OCP FP8 specification, E4M3 column): sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits. Normal values (E = 1..15) are (1 + m/8) * 2^(E-7),
 * subnormals (E = 0) are (m/8) * 2^-6 = m * 2^-9; S.1111.111 is NaN and there
 * is no infinity, so the largest finite magnitude is S.1111.110 = 448.
 * Magnitude codes 0x00..0x7E are ordered like the values they encode.
 */
uint8_t oracle_e4m3fn_from_f32(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  const uint8_t sign = (uint8_t)((u >> 24) & 0x80u);
  const uint32_t mag = u & 0x7FFFFFFFu;

  if (mag > 0x7F800000u) return sign | 0x7Fu; /* NaN */
  if (mag >= 0x43E00000u) return sign | 0x7Eu; /* |f| >= 448, or inf: saturate */

  const int biased = (int)(mag >> 23);      /* fp32 exponent field */
  const uint32_t frac = mag & 0x7FFFFFu;    /* fp32 mantissa field */

  if (biased == 0) return sign; /* fp32 subnormal: far below 2^-10, rounds to 0 */

  const int e = biased - 127; /* |f| = 1.frac * 2^e */

  if (e >= -6) {
    /* Normal E4M3 range: keep 3 of the 23 mantissa bits, RNE on the other 20.
     * A carry out of the mantissa correctly bumps the exponent field. */
    uint32_t code = ((uint32_t)(e + 7) << 3) | (frac >> 20);
    const uint32_t rest = frac & 0xFFFFFu;
    const uint32_t half = 0x80000u;
    if (rest > half || (rest == half && (code & 1u))) code += 1u;
    /* |f| < 448 keeps code <= 0x7E. */
    return sign | (uint8_t)code;
  }

  /* Subnormal E4M3 range: |f| = M * 2^(e-23) with the 24-bit significand M,
   * and the code is k = RNE(|f| / 2^-9) = RNE(M * 2^(e-14)). k = 8 is the
   * smallest normal (0x08), which is the correct code for it. */
  if (e < -17) return sign; /* |f| < 2^-17 < 2^-10 (half of 2^-9): rounds to 0 */
  const uint32_t M = (1u << 23) | frac;
  const int shift = 14 - e; /* 21..31 */
  uint32_t k = M >> shift;
  const uint32_t rest = M & ((1u << shift) - 1u);
  const uint32_t half = 1u << (shift - 1);
  if (rest > half || (rest == half && (k & 1u))) k += 1u;
  return sign | (uint8_t)k;
}

double oracle_e4m3fn_value(uint8_t byte) {
  const int s = byte >> 7;
  const int E = (byte >> 3) & 0xF;
  const int m = byte & 7;
  double v;
  if (E == 15 && m == 7) return NAN;
  if (E == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, E - 7);
  return s ? -v : v;
}

float oracle_tile_scale(float amax) {
  if (amax == 0.0f) return 1.0f;
  return amax / 448.0f; /* IEEE fp32 division */
}

uint8_t oracle_quantize_element(uint16_t x_bits, float s) {
  const float x = oracle_bf16_to_f32(x_bits);
  const float q = x / s; /* IEEE fp32 division, not x * (1/s) */
  return oracle_e4m3fn_from_f32(q);
}

/* Assembly and fusion: the full fused tensor, R x cols, as one buffer.
 * Step 1 rebuilds each component from its shards (the full_tensor() step),
 * step 2 concatenates the components (projection fusion). */
static uint16_t *assemble_and_fuse(const oracle_output *o, int64_t *rows_out) {
  const int64_t C = o->cols;
  int64_t R = 0;
  for (int32_t p = 0; p < o->n_parts; ++p)
    for (int32_t k = 0; k < o->parts[p].n_shards; ++k) R += o->parts[p].shards[k].rows;
  *rows_out = R;

  uint16_t *fused = (uint16_t *)malloc((size_t)(R * C > 0 ? R * C : 1) * sizeof(uint16_t));
  if (!fused) return NULL;

  int64_t fused_row = 0;
  for (int32_t p = 0; p < o->n_parts; ++p) {
    const oracle_part *part = &o->parts[p];
    int64_t Rc = 0;
    for (int32_t k = 0; k < part->n_shards; ++k) Rc += part->shards[k].rows;

    /* Step 1: full component tensor from its shards, in shard order. */
    uint16_t *full = (uint16_t *)malloc((size_t)(Rc * C > 0 ? Rc * C : 1) * sizeof(uint16_t));
    if (!full) {
      free(fused);
      return NULL;
    }
    int64_t row = 0;
    for (int32_t k = 0; k < part->n_shards; ++k) {
      const oracle_shard *sh = &part->shards[k];
      if (sh->rows > 0)
        memcpy(full + row * C, sh->data, (size_t)(sh->rows * C) * sizeof(uint16_t));
      row += sh->rows;
    }

    /* Step 2: append the component below the ones before it. */
    if (Rc > 0) memcpy(fused + fused_row * C, full, (size_t)(Rc * C) * sizeof(uint16_t));
    fused_row += Rc;
    free(full);
  }
  return fused;
}

static int check_output(const oracle_output *o, uint64_t dst_bytes) {
  if (!o || o->cols < 1 || o->n_parts < 1 || !o->parts) return ORACLE_E_ARG;
  if (o->kind != ORACLE_FP8_TILE128 && o->kind != ORACLE_BF16_COPY) return ORACLE_E_ARG;
  int64_t R = 0;
  for (int32_t p = 0; p < o->n_parts; ++p) {
    if (o->parts[p].n_shards < 1 || !o->parts[p].shards) return ORACLE_E_ARG;
    for (int32_t k = 0; k < o->parts[p].n_shards; ++k) {
      const oracle_shard *sh = &o->parts[p].shards[k];
      if (sh->rows < 0 || (sh->rows > 0 && !sh->data)) return ORACLE_E_ARG;
      R += sh->rows;
    }
  }
  if (R < 1) return ORACLE_E_ARG;
  const uint64_t elems = (uint64_t)R * (uint64_t)o->cols;
  const uint64_t data_bytes = o->kind == ORACLE_BF16_COPY ? 2 * elems : elems;
  if (o->dst_offset > dst_bytes || data_bytes > dst_bytes - o->dst_offset) return ORACLE_E_RANGE;
  if (o->kind == ORACLE_FP8_TILE128) {
    const uint64_t tiles = (uint64_t)((R + 127) / 128) * (uint64_t)((o->cols + 127) / 128);
    if (o->scale_offset > dst_bytes || 4 * tiles > dst_bytes - o->scale_offset) return ORACLE_E_RANGE;
  }
  return ORACLE_OK;
}

static int prepare_one(const oracle_output *o, uint8_t *dst, uint64_t dst_bytes) {
  int rc = check_output(o, dst_bytes);
  if (rc != ORACLE_OK) return rc;

  int64_t R = 0;
  const int64_t C = o->cols;
  uint16_t *x = assemble_and_fuse(o, &R);
  if (!x) return ORACLE_E_NOMEM;

  if (o->kind == ORACLE_BF16_COPY) {
    /* Not quantized: the fused BF16 bytes go to the destination unchanged. */
    memcpy(dst + o->dst_offset, x, (size_t)(R * C) * sizeof(uint16_t));
    free(x);
    return ORACLE_OK;
  }

  const int64_t tiles_r = (R + 127) / 128;
  const int64_t tiles_c = (C + 127) / 128;
  uint8_t *q = dst + o->dst_offset;
  uint8_t *scales = dst + o->scale_offset;

  for (int64_t I = 0; I < tiles_r; ++I) {
    for (int64_t J = 0; J < tiles_c; ++J) {
      const int64_t r0 = 128 * I, r1 = (128 * I + 128 < R) ? 128 * I + 128 : R;
      const int64_t c0 = 128 * J, c1 = (128 * J + 128 < C) ? 128 * J + 128 : C;

      /* amax over the tile's valid elements (widening BF16 -> fp32 is exact). */
      float amax = 0.0f;
      for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = c0; c < c1; ++c) {
          const float a = fabsf(oracle_bf16_to_f32(x[r * C + c]));
          if (a > amax) amax = a;
        }

      const float s = oracle_tile_scale(amax);

      for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = c0; c < c1; ++c) q[r * C + c] = oracle_quantize_element(x[r * C + c], s);

      /* Scale grid: row-major over tiles, fp32 little-endian. */
      memcpy(scales + 4 * (I * tiles_c + J), &s, sizeof s);
    }
  }
  free(x);
  return ORACLE_OK;
}

int oracle_prepare(const oracle_output *outs, int64_t n_outs, uint8_t *dst, uint64_t dst_bytes) {
  if (n_outs < 0 || (n_outs > 0 && (!outs || !dst))) return ORACLE_E_ARG;
  for (int64_t i = 0; i < n_outs; ++i) {
    int rc = prepare_one(&outs[i], dst, dst_bytes);
    if (rc != ORACLE_OK) return rc;
  }
  return ORACLE_OK;
}

void oracle_quantize_domain(const uint16_t *amax_bits, int64_t n_amax, uint8_t *out) {
  for (int64_t i = 0; i < n_amax; ++i) {
    const float s = oracle_tile_scale(oracle_bf16_to_f32(amax_bits[i]));
    for (uint32_t xb = 0; xb < 65536u; ++xb)
      out[i * 65536 + xb] = oracle_quantize_element((uint16_t)xb, s);
  }
}

void oracle_cast_f32_range(uint32_t first, uint64_t count, uint8_t *out) {
  for (uint64_t i = 0; i < count; ++i) {
    const uint32_t bits = first + (uint32_t)i;
    float f;
    memcpy(&f, &bits, sizeof f);
    out[i] = oracle_e4m3fn_from_f32(f);
  }
}

void oracle_cast_f32_array(const float *in, int64_t n, uint8_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3fn_from_f32(in[i]);
}

void oracle_quantize_elements(const uint16_t *x_bits, int64_t n, float s, uint8_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_quantize_element(x_bits[i], s);
}

int oracle_quantize_act_b128(const uint16_t *x, int64_t n_rows, int64_t cols, int64_t x_stride,
                             const int32_t *index, int64_t n_out, uint8_t *q, int64_t q_stride,
                             uint8_t *scales, int64_t s_stride) {
  if (n_rows < 0 || cols < 1 || n_out < 0 || x_stride < cols || q_stride < cols) return ORACLE_E_ARG;
  const int64_t nb = (cols + 127) / 128;
  if (s_stride < 4 * nb) return ORACLE_E_ARG;
  if (n_out > 0 && (!q || !scales || (n_rows > 0 && !x))) return ORACLE_E_ARG;
  for (int64_t i = 0; i < n_out; ++i) {
    const int64_t src = index ? (int64_t)index[i] : i;
    if (src < 0 || src >= n_rows) continue;
    const uint16_t *xr = x + src * x_stride;
    for (int64_t b = 0; b < nb; ++b) {
      const int64_t c0 = 128 * b, c1 = (c0 + 128 < cols) ? c0 + 128 : cols;
      float amax = 0.0f;
      for (int64_t c = c0; c < c1; ++c) {
        const float a = fabsf(oracle_bf16_to_f32(xr[c]));
        if (a > amax) amax = a;
      }
      const float s = oracle_tile_scale(amax);
      for (int64_t c = c0; c < c1; ++c) q[i * q_stride + c] = oracle_quantize_element(xr[c], s);
      memcpy(scales + i * s_stride + 4 * b, &s, sizeof s);
    }
  }
  return ORACLE_OK;
}
