// act_quant.hip -- block-scaled FP8 quantization of token activations
// ("Enabling trillion-parameter models on AWS EFA", dispatch/combine
// evaluation: hidden size 7168, FP8 dispatch with block scales). A block is
// one token's 128 consecutive channels (the last block of a row may be
// shorter); per block s = amax / 448 (1 for an all-zero block) and
// q = cast(fl32(x / s)) with the same element arithmetic as the weight tiles.
// Output row i quantizes input row index[i] (row i without an index), which
// fuses the sender's shuffle of tokens into send-buffer slots with the
// quantization; rows whose index is out of range are skipped.
//
// Mapping: one 16-lane DPP row per block, lane l owns channels
// [128 b + 8 l, +8): one 16-byte load and one 8-byte store per lane, so a
// wave reads four blocks (1 KB) and writes 512 bytes per instruction. The
// block's amax is a butterfly max over the 16 lanes (quad_perm, row half
// mirror, row mirror), which leaves it in every lane of the row.
#include <hip/hip_runtime.h>

#include "fp8_math.h"
#include "wt_internal.h"

namespace wt {
namespace {

#ifndef WT_ACT_THREADS
#define WT_ACT_THREADS 256
#endif
#ifndef WT_ACT_K
#define WT_ACT_K 1
#endif
// Cache hints, measured on MI355X for 4096 x 7168 (us per launch, back to
// back): plain 16.47, non-temporal stores 16.94, non-temporal loads 18.84,
// both 17.52. Plain accesses stay the default.
#ifndef WT_ACT_NT_LOAD
#define WT_ACT_NT_LOAD 0
#endif
#ifndef WT_ACT_NT_STORE
#define WT_ACT_NT_STORE 0
#endif
typedef unsigned int act_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int act_u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 act_load16(uint64_t a) {
#if defined(__HIP_DEVICE_COMPILE__)
  if (WT_ACT_NT_LOAD) {
    const act_u32x4 v = __builtin_nontemporal_load((const __attribute__((address_space(1))) act_u32x4 *)(uintptr_t)a);
    return make_uint4(v.x, v.y, v.z, v.w);
  }
#endif
  return ld_global<uint4>(a);
}

__device__ __forceinline__ void act_store8(uint64_t a, uint2 q) {
#if defined(__HIP_DEVICE_COMPILE__)
  if (WT_ACT_NT_STORE) {
    act_u32x2 v;
    v.x = q.x;
    v.y = q.y;
    __builtin_nontemporal_store(v, (__attribute__((address_space(1))) act_u32x2 *)(uintptr_t)a);
    return;
  }
#endif
  st_global<uint2>(a, q);
}
constexpr int kActThreads = WT_ACT_THREADS;
constexpr int kActGroups = kActThreads / 16;  // 16-lane groups per workgroup
constexpr int kActK = WT_ACT_K;               // blocks per group (loads in flight per lane)

__device__ __forceinline__ uint32_t row16_max(uint32_t m) {
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x0B1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x04E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x141, 0xF, 0xF, false));  // row_half_mirror
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x140, 0xF, 0xF, false));  // row_mirror
  return m;
}

template <bool Recip>
__device__ __forceinline__ uint2 quant8(const uint32_t w[4], const TileQ &t) {
  return make_uint2(quant4<Recip>(w[0], w[1], t), quant4<Recip>(w[2], w[3], t));
}

// Where block gblk of the launch lives: its output row, block column and
// source row; has = this lane holds channels of it.
struct BlockAt {
  uint32_t i, b;
  int64_t src, c;
  bool has;
};

__device__ __forceinline__ BlockAt locate(const ActArgs &a, uint32_t gblk, uint32_t l) {
  BlockAt p{0, 0, -1, 0, false};
  if (gblk < a.n_blocks) {
    p.i = gblk / a.nb;
    p.b = gblk - p.i * a.nb;
    p.src = a.index ? (int64_t)ld_global<int32_t>(a.index + 4ull * p.i) : (int64_t)p.i;
    p.c = 128 * (int64_t)p.b + 8 * (int64_t)l;
    p.has = p.src >= 0 && p.src < a.n_rows && p.c < a.cols;
  }
  return p;
}

// Fast: cols, x_stride, q_stride multiples of 8, x 16-byte and q 8-byte
// aligned; each group takes K blocks, all K loads issued before any use.
// General (K = 1): any shape and alignment (2-byte loads, byte stores).
template <bool Fast, int K>
__global__ void __launch_bounds__(kActThreads) act_quant_kernel(ActArgs a) {
  const uint32_t l = threadIdx.x & 15;
  const uint32_t base = blockIdx.x * (uint32_t)(kActGroups * K) + (threadIdx.x >> 4);
  BlockAt p[K];
  uint32_t w[K][4];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    p[k] = locate(a, base + (uint32_t)(k * kActGroups), l);
    w[k][0] = w[k][1] = w[k][2] = w[k][3] = 0u;
    const uint64_t xrow = a.x + 2ull * (uint64_t)p[k].src * (uint64_t)a.x_stride;
    if (Fast) {
      if (p[k].has) {
        const uint4 v = act_load16(xrow + 2ull * (uint64_t)p[k].c);
        w[k][0] = v.x, w[k][1] = v.y, w[k][2] = v.z, w[k][3] = v.w;
      }
    } else if (p[k].has) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (p[k].c + e < a.cols)
          w[k][e >> 1] |= (uint32_t)ld_global<uint16_t>(xrow + 2ull * (uint64_t)(p[k].c + e)) << (16 * (e & 1));
    }
  }
#pragma unroll
  for (int k = 0; k < K; ++k) {
    uint32_t m = pk_max_u16(pk_max_u16(abs2(w[k][0]), abs2(w[k][1])), pk_max_u16(abs2(w[k][2]), abs2(w[k][3])));
    m = row16_max(max(m & 0xFFFFu, m >> 16));  // every lane of the row takes part
    if (p[k].has) {
      const TileQ t = block_quant(m);
      const uint64_t qrow = a.q + (uint64_t)p[k].i * (uint64_t)a.q_stride;
      if (Fast) {
        const uint2 q = t.recip ? quant8<true>(w[k], t) : quant8<false>(w[k], t);
        act_store8(qrow + (uint64_t)p[k].c, q);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (p[k].c + e < a.cols) {
            const uint32_t xb = (w[k][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
            const uint32_t q = t.recip ? quant1<true>(xb, t) : quant1<false>(xb, t);
            st_global<uint8_t>(qrow + (uint64_t)(p[k].c + e), (uint8_t)q);
          }
      }
      if (l == 0) st_global<float>(a.s + (uint64_t)p[k].i * (uint64_t)a.s_stride + 4ull * p[k].b, t.s);
    }
  }
}

}  // namespace

hipError_t launch_act_quant(const ActArgs &a, bool fast, hipStream_t stream) {
  if (a.n_blocks == 0) return hipSuccess;
  if (fast) {
    const dim3 grid((a.n_blocks + kActGroups * kActK - 1) / (kActGroups * kActK));
    hipLaunchKernelGGL((act_quant_kernel<true, kActK>), grid, dim3(kActThreads), 0, stream, a);
  } else {
    const dim3 grid((a.n_blocks + kActGroups - 1) / kActGroups);
    hipLaunchKernelGGL((act_quant_kernel<false, 1>), grid, dim3(kActThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace wt
