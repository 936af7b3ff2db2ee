// fp8_math.h -- device-side element arithmetic shared by the weight-tile and
// activation-block kernels: global/constant address-space access helpers,
// packed-BF16 magnitude max, the block scale s = amax / 448, the division
// x / s (reciprocal with an exact correction, or IEEE division), and the
// saturating round-to-nearest-even cast to OCP E4M3 ("e4m3fn"). The
// per-element code is exactly what wt_quantize_domain checks over every
// (x, amax) pair of BF16.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace wt {

// ------------------------------------------------------------ memory access
// Descriptor tables are read-only for the kernel's lifetime and read at
// workgroup-uniform addresses: constant address space, so they become scalar
// loads. Tensor data goes through the global address space (global_load /
// global_store rather than flat instructions, which would also count against
// the LDS counter).
template <class T>
using cptr = const __attribute__((address_space(4))) T *;
template <class T>
using gptr = __attribute__((address_space(1))) T *;
template <class T>
using gcptr = const __attribute__((address_space(1))) T *;

// p[i] from a descriptor table (scalar load when i is uniform).
template <class T>
__device__ __forceinline__ T ld_table(const T *p, uint64_t i) {
#if defined(__HIP_DEVICE_COMPILE__)
  return ((cptr<T>)(uintptr_t)p)[i];
#else
  return p[i];
#endif
}
// Global-memory load / store at a byte address.
template <class T>
__device__ __forceinline__ T ld_global(uint64_t a) {
#if defined(__HIP_DEVICE_COMPILE__)
  return *(gcptr<T>)(uintptr_t)a;
#else
  return *(const T *)(uintptr_t)a;
#endif
}
template <class T>
__device__ __forceinline__ void st_global(uint64_t a, const T &v) {
#if defined(__HIP_DEVICE_COMPILE__)
  *(gptr<T>)(uintptr_t)a = v;
#else
  *(T *)(uintptr_t)a = v;
#endif
}

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

// Division x / s for one tile. For tiles with s >= 2^-100 the quotient is
// computed from the tile's correctly rounded reciprocal r = 1/s with one
// exact residual (Markstein's correction, Handbook of Floating-Point
// Arithmetic, section on division with FMA): y = x*r, d = y*s - x (exact in
// one FMA), q = y - d*r. The residual is arranged as y*s - x (not x - y*s)
// so that signed zeros come out as IEEE division gives them. Below the
// threshold (amax < about 448 * 2^-100) intermediate products can be
// subnormal and the tile uses the compiler's IEEE division. Which form is
// used is one uniform decision per tile; the complete (x, amax) domain of
// BF16 is checked against IEEE division by wt_quantize_domain.
#ifndef WT_RECIP_DIV
#define WT_RECIP_DIV 1
#endif

struct TileQ {
  float s;  // the tile's scale
  float r;  // fl(1 / s), used when recip
  bool recip;
};

// Scale, reciprocal and division form of one block; s >= 2^-100 selects the
// reciprocal form.
__device__ __forceinline__ TileQ block_quant(uint32_t amax16) {
  TileQ t;
  t.s = tile_scale(amax16);
  t.r = 1.0f / t.s;
  t.recip = WT_RECIP_DIV && __float_as_uint(t.s) >= 0x0D800000u;
  return t;
}

// The same for a block whose amax every lane of the wave holds: the choice
// becomes one uniform branch.
__device__ __forceinline__ TileQ tile_quant(uint32_t amax16) {
  TileQ t = block_quant(amax16);
  t.recip = __builtin_amdgcn_readfirstlane(t.recip);
  return t;
}

template <bool Recip>
__device__ __forceinline__ float qdiv(float x, const TileQ &t) {
  if (Recip) {
    const float y = x * t.r;
    const float d = __builtin_fmaf(y, t.s, -x);
    return __builtin_fmaf(-d, t.r, y);
  }
  return x / t.s;
}

// Saturation to [-448, 448] (v_cvt_pk_fp8_f32 rounds to nearest even but
// does not saturate: from 464 up it gives the NaN code, and it takes no clamp
// modifier). Used by the standalone cast check (cast of any fp32 value).
__device__ __forceinline__ float sat448(float q) { return __builtin_amdgcn_fmed3f(q, -448.0f, 448.0f); }

// The element functions below convert without that clamp: a block's
// quotients are |x| / s <= amax / s, at most 448.88 in magnitude for every
// positive BF16 amax (448 exactly up to the rounding of s), and the convert
// rounds every value below 464 to at most 448 (0x7E) on its own, so a clamp
// could never change a byte. wt_quantize_domain runs exactly this code over
// every (x, amax) pair of BF16 values with |x| <= amax, which is how the
// claim is checked against the oracle's saturating cast.

// Four BF16 (two packed words) -> four E4M3 bytes, little-endian in one word.
template <bool Recip>
__device__ __forceinline__ uint32_t quant4(uint32_t w0, uint32_t w1, const TileQ &t) {
  const float a = qdiv<Recip>(bf16_lo(w0), t), b = qdiv<Recip>(bf16_hi(w0), t);
  const float c = qdiv<Recip>(bf16_lo(w1), t), d = qdiv<Recip>(bf16_hi(w1), t);
  // the first convert fills bytes 0-1 and keeps bytes 2-3 of its third
  // operand, which the second convert then overwrites: any register will do
  uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)w1, false);
  r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)r, true);
  return r;
}

// Two packed BF16 -> two E4M3 bytes in bits 0-7 (low half) and 8-15 (high
// half); bits 16-31 are left over from the input. Same arithmetic as quant4.
template <bool Recip>
__device__ __forceinline__ uint32_t quant2(uint32_t w, const TileQ &t) {
  const float a = qdiv<Recip>(bf16_lo(w), t), b = qdiv<Recip>(bf16_hi(w), t);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)w, false);
}

// One BF16 -> one E4M3 byte (same arithmetic as quant4, one lane).
template <bool Recip>
__device__ __forceinline__ uint32_t quant1(uint32_t xbits, const TileQ &t) {
  const float a = qdiv<Recip>(__uint_as_float(xbits << 16), t);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, 0.0f, 0, false) & 0xFFu;
}

}  // namespace wt
