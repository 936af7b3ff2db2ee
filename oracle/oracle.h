/*
 * oracle.h -- plain CPU reference for the parameter-preparation stage.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may include, link,
 * load or call this code: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no source, header, table or helper with
 * the GPU library; the two meet only through identical input bytes.
 *
 * What is computed ("Weight transfer for RL post-training in under 2
 * seconds", Perplexity, section "Task pipeline": parameter preparation
 * rebuilds the full weight with full_tensor(), applies projection fusion, and
 * quantizes if needed; section "DeviceMesh and mesh groups": parameters are
 * placed by FSDP). The page fixes none of the numerics; the readings taken
 * here are:
 *   - FSDP placement = dim-0 row shards; assembly = concatenation of the
 *     shards' rows in shard order;
 *   - projection fusion = dim-0 concatenation of the component tensors in
 *     the order given (q, k, v; gate, up);
 *   - "quantize" = OCP FP8 E4M3 ("e4m3fn": bias 7, max 448, no infinity,
 *     NaN = S.1111.111) with one fp32 scale per 128x128 tile of the fused
 *     tensor, s = amax / 448 (s = 1 for an all-zero tile), per element
 *     q = fl32(x / s) followed by round-to-nearest-even with saturation
 *     to +-448. Both roundings are part of the definition, so the
 *     arithmetic is fp32 on purpose (the stored scale is fp32 and the
 *     quotient is an fp32 value before the cast); computing in fp64 would
 *     give a different result, not a more exact one.
 *   - tensors that are not quantized are copied byte for byte (BF16).
 *   - FP8 bytes are stored row-major at dst_offset; scales row-major over
 *     the ceil(R/128) x ceil(C/128) tile grid, fp32 little-endian, at
 *     scale_offset.
 */
#ifndef WT_ORACLE_H
#define WT_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_FP8_TILE128 = 0, ORACLE_BF16_COPY = 1 };

enum {
  ORACLE_OK = 0,
  ORACLE_E_ARG = -1,   /* malformed description (null pointer, negative size) */
  ORACLE_E_RANGE = -2, /* an output range falls outside the destination image */
  ORACLE_E_NOMEM = -3
};

/* One FSDP shard: `rows` consecutive rows of a row-major BF16 tensor whose
 * row length is the output's `cols`. rows may be 0. */
typedef struct {
  const uint16_t *data;
  int64_t rows;
} oracle_shard;

/* One source tensor (a fusion component) given as its shards in rank order. */
typedef struct {
  const oracle_shard *shards;
  int32_t n_shards;
} oracle_part;

/* One output tensor: the components in fusion order, all with `cols`
 * columns. For ORACLE_BF16_COPY the scale_offset is ignored. */
typedef struct {
  const oracle_part *parts;
  int32_t n_parts;
  int32_t kind;
  int64_t cols;
  uint64_t dst_offset;
  uint64_t scale_offset;
} oracle_output;

/* BF16 bit pattern -> fp32 (exact widening). */
float oracle_bf16_to_f32(uint16_t bits);

/* fp32 -> OCP E4M3 byte, round to nearest, ties to even, saturating:
 * |f| >= 448 (and +-inf) -> S.1111.110, NaN -> S.1111.111, sign kept for
 * zero and underflow. */
uint8_t oracle_e4m3fn_from_f32(float f);

/* Exact value of an E4M3 byte as a double (NaN for S.1111.111). */
double oracle_e4m3fn_value(uint8_t byte);

/* Tile scale from the tile's amax: amax / 448 in fp32, or 1 when amax == 0. */
float oracle_tile_scale(float amax);

/* One element: cast(fl32(x / s)). */
uint8_t oracle_quantize_element(uint16_t x_bits, float s);

/* Prepares every output into the host image `dst` of dst_bytes bytes.
 * Bytes outside the outputs' ranges are left untouched. */
int oracle_prepare(const oracle_output *outs, int64_t n_outs, uint8_t *dst,
                   uint64_t dst_bytes);

/* For each amax (a BF16 bit pattern) and each of the 65,536 BF16 patterns x:
 * out[i * 65536 + x] = oracle_quantize_element(x, oracle_tile_scale(amax_i)). */
void oracle_quantize_domain(const uint16_t *amax_bits, int64_t n_amax, uint8_t *out);

/* out[i] = oracle_e4m3fn_from_f32(bit pattern first + i), i < count. */
void oracle_cast_f32_range(uint32_t first, uint64_t count, uint8_t *out);

/* out[i] = oracle_e4m3fn_from_f32(in[i]). */
void oracle_cast_f32_array(const float *in, int64_t n, uint8_t *out);

/* out[i] = oracle_quantize_element(x_bits[i], s). */
void oracle_quantize_elements(const uint16_t *x_bits, int64_t n, float s, uint8_t *out);

/* Block-scaled FP8 quantization of token activations ("Enabling
 * trillion-parameter models on AWS EFA", dispatch/combine evaluation: hidden
 * size 7168, FP8 dispatch with block scales). Readings: a block is 1 x 128
 * (one token, 128 consecutive channels; the last block of a row holds the
 * remaining cols % 128 channels), with the weight tiles' scale and element
 * arithmetic. Output row i quantizes input row index[i] (row i when index is
 * NULL); an output row whose index lies outside [0, n_rows) is left
 * untouched. x: n_rows rows of x_stride BF16 elements (the first cols used).
 * q: n_out rows of q_stride bytes, the row's cols FP8 bytes first. scales:
 * n_out rows of s_stride bytes, the row's ceil(cols / 128) fp32 scales first.
 * Bytes past cols (q) and past the scales (scales) are left untouched. */
int oracle_quantize_act_b128(const uint16_t *x, int64_t n_rows, int64_t cols, int64_t x_stride,
                             const int32_t *index, int64_t n_out, uint8_t *q, int64_t q_stride,
                             uint8_t *scales, int64_t s_stride);

#ifdef __cplusplus
}
#endif

#endif
