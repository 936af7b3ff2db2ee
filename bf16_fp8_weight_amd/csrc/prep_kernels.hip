// prep_kernels.hip -- CDNA4 (gfx950) kernels of the parameter-preparation
// stage ("Weight transfer for RL post-training in under 2 seconds", section
// "Task pipeline": rebuild the full weight from its FSDP shards, fuse
// projections, quantize). Assembly and fusion are virtual: a tile reads its
// rows straight from the shard buffers through the row-segment table, so no
// full tensor is ever materialised. Per 128 x 128 tile of an FP8 output:
// amax of |x|, s = amax / 448 (1 for an all-zero tile), q = fl32(x / s) with
// IEEE division, then E4M3 (OCP "e4m3fn") round-to-nearest-even with
// saturation, stored row-major with the fp32 scale at its grid position.
// BF16 pass-through outputs are byte copies. The path is HBM-bound: every
// input byte is read once and every output byte written once.
#include <hip/hip_runtime.h>

#include "wt_internal.h"

namespace wt {

// ------------------------------------------------------------ element math

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}

// |x| of two packed BF16 values, as two 15-bit magnitudes (finite BF16
// compare like their magnitude bits).
__device__ __forceinline__ uint32_t abs2(uint32_t w) { return w & 0x7FFF7FFFu; }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Tile scale from the BF16 magnitude bits of the tile's amax: amax / 448 in
// IEEE fp32 (denormals kept), or 1 for an all-zero tile.
__device__ __forceinline__ float tile_scale(uint32_t amax16) {
  if (amax16 == 0) return 1.0f;
  return __uint_as_float(amax16 << 16) / 448.0f;
}

// Saturation to the E4M3 range before the hardware convert; together with
// round-to-nearest-even in v_cvt_pk_fp8_f32 this gives the saturating cast.
__device__ __forceinline__ float sat448(float q) { return __builtin_amdgcn_fmed3f(q, -448.0f, 448.0f); }

// Four BF16 (two packed words) -> four E4M3 bytes, little-endian in one word.
__device__ __forceinline__ uint32_t quant4(uint32_t w0, uint32_t w1, float s) {
  const float a = bf16_lo(w0) / s, b = bf16_hi(w0) / s;
  const float c = bf16_lo(w1) / s, d = bf16_hi(w1) / s;
  uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
  r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), (int)r, true);
  return r;
}

// One BF16 -> one E4M3 byte (same arithmetic as quant4, one lane).
__device__ __forceinline__ uint32_t quant1(uint32_t xbits, float s) {
  const float a = __uint_as_float(xbits << 16) / s;
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), 0.0f, 0, false) & 0xFFu;
}

// Max over the workgroup (4 waves). red: 4 words of LDS.
__device__ __forceinline__ uint32_t block_max(uint32_t m, uint32_t *red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = m;
  __syncthreads();
  return max(max(red[0], red[1]), max(red[2], red[3]));
}

// ------------------------------------------------------------ tile: fast path
// cols % 8 == 0, 16-byte aligned rows, 8-byte aligned FP8 rows. Thread t
// owns 8 columns (16 bytes of BF16) of rows (t >> 4) + 16 k, k = 0..7: a
// wave reads four full 256-byte tile rows per instruction and writes four
// 128-byte FP8 rows per store. The 64 values stay in registers between the
// amax and the quantization.
__device__ __forceinline__ void fast_tile(const LaunchTables &T, const TileItem it, uint32_t *red) {
  const DevOut o = T.outs[it.out];
  const int tid = threadIdx.x;
  const int cc = tid & 15;
  const int rr = tid >> 4;
  const int64_t r0 = (int64_t)it.tile_row * kTile;
  const int64_t rlim = min(r0 + (int64_t)kTile, o.rows);
  const int64_t c = (int64_t)it.tile_col * kTile + cc * 8;
  const bool col_ok = c < o.cols;
  const int64_t C = o.cols;

  uint4 v[8];
  uint32_t idx = it.seg;
  DevSeg g = T.segs[idx];
  const bool single = g.row_end >= rlim;  // uniform: one shard serves the whole tile row
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int64_t r = r0 + rr + 16 * k;
    v[k] = make_uint4(0, 0, 0, 0);
    if (col_ok && r < rlim) {
      if (!single)
        while (r >= g.row_end) g = T.segs[++idx];
      const uint4 *p = reinterpret_cast<const uint4 *>(g.src + (uint64_t)(((r - g.row0) * C + c) * 2));
      v[k] = *p;
    }
  }

  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    m = pk_max_u16(m, abs2(v[k].x));
    m = pk_max_u16(m, abs2(v[k].y));
    m = pk_max_u16(m, abs2(v[k].z));
    m = pk_max_u16(m, abs2(v[k].w));
  }
  m = max(m & 0xFFFFu, m >> 16);
  const uint32_t amax16 = block_max(m, red);
  const float s = tile_scale(amax16);

#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int64_t r = r0 + rr + 16 * k;
    if (col_ok && r < rlim) {
      uint2 q;
      q.x = quant4(v[k].x, v[k].y, s);
      q.y = quant4(v[k].z, v[k].w, s);
      *reinterpret_cast<uint2 *>(o.q + (uint64_t)(r * C + c)) = q;
    }
  }
  if (tid == 0) reinterpret_cast<float *>(o.s)[(uint64_t)it.tile_row * (uint64_t)o.tiles_c + it.tile_col] = s;
}

// ------------------------------------------------------------ tile: general path
// Any cols and alignment. Thread t owns column t & 127 of rows (t >> 7) + 2 k.
// Pass 1 reads the tile for its amax, pass 2 reads it again (now from cache)
// and quantizes; 2-byte loads and 1-byte stores, coalesced along each row.
__device__ __forceinline__ void general_tile(const LaunchTables &T, const TileItem it, uint32_t *red) {
  const DevOut o = T.outs[it.out];
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)it.tile_row * kTile;
  const int64_t rlim = min(r0 + (int64_t)kTile, o.rows);
  const int64_t c = (int64_t)it.tile_col * kTile + (tid & 127);
  const bool col_ok = c < o.cols;
  const int64_t C = o.cols;
  const int rb = tid >> 7;

  uint32_t m = 0;
  {
    uint32_t idx = it.seg;
    DevSeg g = T.segs[idx];
    for (int k = 0; k < kTile / 2; ++k) {
      const int64_t r = r0 + rb + 2 * k;
      if (!col_ok || r >= rlim) break;
      while (r >= g.row_end) g = T.segs[++idx];
      const uint16_t x = *reinterpret_cast<const uint16_t *>(g.src + (uint64_t)(((r - g.row0) * C + c) * 2));
      m = max(m, (uint32_t)(x & 0x7FFFu));
    }
  }
  const uint32_t amax16 = block_max(m, red);
  const float s = tile_scale(amax16);
  {
    uint32_t idx = it.seg;
    DevSeg g = T.segs[idx];
    for (int k = 0; k < kTile / 2; ++k) {
      const int64_t r = r0 + rb + 2 * k;
      if (!col_ok || r >= rlim) break;
      while (r >= g.row_end) g = T.segs[++idx];
      const uint16_t x = *reinterpret_cast<const uint16_t *>(g.src + (uint64_t)(((r - g.row0) * C + c) * 2));
      *reinterpret_cast<uint8_t *>(o.q + (uint64_t)(r * C + c)) = (uint8_t)quant1(x, s);
    }
  }
  if (tid == 0) reinterpret_cast<float *>(o.s)[(uint64_t)it.tile_row * (uint64_t)o.tiles_c + it.tile_col] = s;
}

// ------------------------------------------------------------ pass-through copy
// One wave per item; src, dst and bytes are multiples of width.
__device__ __forceinline__ void copy_item(const CopyItem ci, int lane) {
  switch (ci.width) {
    case 16: {
      const uint4 *s = reinterpret_cast<const uint4 *>(ci.src);
      uint4 *d = reinterpret_cast<uint4 *>(ci.dst);
      for (uint32_t i = lane; i < ci.bytes / 16; i += 64) d[i] = s[i];
      break;
    }
    case 4: {
      const uint32_t *s = reinterpret_cast<const uint32_t *>(ci.src);
      uint32_t *d = reinterpret_cast<uint32_t *>(ci.dst);
      for (uint32_t i = lane; i < ci.bytes / 4; i += 64) d[i] = s[i];
      break;
    }
    case 2: {
      const uint16_t *s = reinterpret_cast<const uint16_t *>(ci.src);
      uint16_t *d = reinterpret_cast<uint16_t *>(ci.dst);
      for (uint32_t i = lane; i < ci.bytes / 2; i += 64) d[i] = s[i];
      break;
    }
    default: {
      const uint8_t *s = reinterpret_cast<const uint8_t *>(ci.src);
      uint8_t *d = reinterpret_cast<uint8_t *>(ci.dst);
      for (uint32_t i = lane; i < ci.bytes; i += 64) d[i] = s[i];
      break;
    }
  }
}

// ------------------------------------------------------------ kernels

// Blocks [0, n_fast): one fast tile each; then kCopiesPerBlock copy items per block.
__global__ __launch_bounds__(kBlock) void prep_fast_copy_kernel(LaunchTables T) {
  __shared__ uint32_t red[4];
  const uint32_t b = blockIdx.x;
  if (b < T.n_fast) {
    fast_tile(T, T.fast_tiles[b], red);
    return;
  }
  const uint32_t ci = (b - T.n_fast) * kCopiesPerBlock + (threadIdx.x >> 6);
  if (ci < T.n_copies) copy_item(T.copies[ci], threadIdx.x & 63);
}

__global__ __launch_bounds__(kBlock) void prep_general_kernel(LaunchTables T) {
  __shared__ uint32_t red[4];
  general_tile(T, T.general_tiles[blockIdx.x], red);
}

// Element-function check: out[i * 65536 + x] for every BF16 x, four per thread,
// through the same tile_scale / quant4 as the fast tile path.
__global__ __launch_bounds__(kBlock) void quantize_domain_kernel(const uint16_t *amax_bits, int64_t n_amax,
                                                                 uint8_t *out) {
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int64_t i = gid >> 14;
  if (i >= n_amax) return;
  const uint32_t x0 = (uint32_t)(gid & 16383) * 4;
  const float s = tile_scale(amax_bits[i] & 0x7FFFu);
  const uint32_t w0 = x0 | ((x0 + 1) << 16);
  const uint32_t w1 = (x0 + 2) | ((x0 + 3) << 16);
  *reinterpret_cast<uint32_t *>(out + i * 65536 + x0) = quant4(w0, w1, s);
}

// The same domain through quant1 (the general tile path's element function).
__global__ __launch_bounds__(kBlock) void quantize_domain1_kernel(const uint16_t *amax_bits, int64_t n_amax,
                                                                  uint8_t *out) {
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int64_t i = gid >> 16;
  if (i >= n_amax) return;
  const uint32_t x = (uint32_t)(gid & 65535);
  const float s = tile_scale(amax_bits[i] & 0x7FFFu);
  out[i * 65536 + x] = (uint8_t)quant1(x, s);
}

// Cast check: the saturating E4M3 cast of fp32 patterns first + i.
__global__ __launch_bounds__(kBlock) void cast_range_kernel(uint32_t first, uint64_t count, uint8_t *out) {
  const uint64_t i = ((uint64_t)blockIdx.x * kBlock + threadIdx.x) * 4;
  if (i >= count) return;
  float f[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) f[k] = __uint_as_float(first + (uint32_t)(i + k));
  uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat448(f[0]), sat448(f[1]), 0, false);
  r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat448(f[2]), sat448(f[3]), (int)r, true);
  if (i + 4 <= count) {
    *reinterpret_cast<uint32_t *>(out + i) = r;
  } else {
    for (uint64_t k = 0; i + k < count; ++k) out[i + k] = (uint8_t)(r >> (8 * k));
  }
}

// ------------------------------------------------------------ launchers

hipError_t launch_batch(const LaunchTables &T, hipStream_t stream) {
  const uint64_t copy_blocks = (T.n_copies + kCopiesPerBlock - 1) / kCopiesPerBlock;
  const uint64_t blocks = (uint64_t)T.n_fast + copy_blocks;
  if (blocks > 0) {
    hipLaunchKernelGGL(prep_fast_copy_kernel, dim3((uint32_t)blocks), dim3(kBlock), 0, stream, T);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (T.n_general > 0) {
    hipLaunchKernelGGL(prep_general_kernel, dim3(T.n_general), dim3(kBlock), 0, stream, T);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_quantize_domain(const uint16_t *amax_bits, int64_t n_amax, uint8_t *out, int variant,
                                  hipStream_t stream) {
  if (n_amax <= 0) return hipSuccess;
  if (variant == 0) {
    const uint64_t blocks = (uint64_t)n_amax * 16384 / kBlock;
    hipLaunchKernelGGL(quantize_domain_kernel, dim3((uint32_t)blocks), dim3(kBlock), 0, stream, amax_bits, n_amax,
                       out);
  } else {
    const uint64_t blocks = (uint64_t)n_amax * 65536 / kBlock;
    hipLaunchKernelGGL(quantize_domain1_kernel, dim3((uint32_t)blocks), dim3(kBlock), 0, stream, amax_bits, n_amax,
                       out);
  }
  return hipGetLastError();
}

hipError_t launch_cast_range(uint32_t first, uint64_t count, uint8_t *out, hipStream_t stream) {
  if (count == 0) return hipSuccess;
  const uint64_t threads = (count + 3) / 4;
  const uint64_t blocks = (threads + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(cast_range_kernel, dim3((uint32_t)blocks), dim3(kBlock), 0, stream, first, count, out);
  return hipGetLastError();
}

}  // namespace wt
