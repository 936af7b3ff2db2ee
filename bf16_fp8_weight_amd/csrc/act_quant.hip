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
// Mapping, aligned rows: eight lanes per block, lane l owning the block's
// 16-byte chunks l and l + 8, so each load and store instruction covers
// consecutive bytes across a wave and a wave holds eight blocks; the block's
// amax is a DPP max over its eight lanes. Unaligned rows: one 16-lane DPP row
// per block, 2-byte loads and byte stores.
#include <hip/hip_runtime.h>

#include "fp8_math.h"
#include "wt_internal.h"

namespace wt {
namespace {

#ifndef WT_ACT_THREADS
#define WT_ACT_THREADS 256
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
constexpr int kActGroups = kActThreads / 16;  // 16-lane groups per workgroup (unaligned path)

// Max over the L lanes of each aligned L-lane group (DPP within 16-lane rows;
// lanes read from outside the group take no part), left in every lane.
template <int L>
__device__ __forceinline__ uint32_t lanes_max(uint32_t m) {
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x0B1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x04E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
  if (L >= 8) m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x141, 0xF, 0xF, false));  // row_half_mirror
  if (L >= 16) m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x140, 0xF, 0xF, false));  // row_mirror
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

// Unaligned path (any shape and alignment): one block per 16-lane group, lane
// l owns channels [128 b + 8 l, +8), read with 2-byte loads and written with
// byte stores.
__global__ void __launch_bounds__(kActThreads) act_quant_kernel(ActArgs a) {
  const uint32_t l = threadIdx.x & 15;
  const BlockAt p = locate(a, blockIdx.x * (uint32_t)kActGroups + (threadIdx.x >> 4), l);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  const uint64_t xrow = a.x + 2ull * (uint64_t)p.src * (uint64_t)a.x_stride;
  if (p.has) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (p.c + e < a.cols)
        w[e >> 1] |= (uint32_t)ld_global<uint16_t>(xrow + 2ull * (uint64_t)(p.c + e)) << (16 * (e & 1));
  }
  uint32_t m = pk_max_u16(pk_max_u16(abs2(w[0]), abs2(w[1])), pk_max_u16(abs2(w[2]), abs2(w[3])));
  m = lanes_max<16>(max(m & 0xFFFFu, m >> 16));  // every lane of the row takes part
  if (!p.has) return;
  const TileQ t = block_quant(m);
  const uint64_t qrow = a.q + (uint64_t)p.i * (uint64_t)a.q_stride;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (p.c + e < a.cols) {
      const uint32_t xb = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      const uint32_t q = t.recip ? quant1<true>(xb, t) : quant1<false>(xb, t);
      st_global<uint8_t>(qrow + (uint64_t)(p.c + e), (uint8_t)q);
    }
  if (l == 0) st_global<float>(a.s + (uint64_t)p.i * (uint64_t)a.s_stride + 4ull * p.b, t.s);
}

// Lanes per block on the aligned path: each lane owns 128 / L channels
// (128 / (8 L) 16-byte chunks), so the per-block work (locating the block,
// its scale and reciprocal, the lane reduction) is paid once per 128 / L
// elements of each lane instead of once per 8.
// Measured on MI355X (us per launch back to back; 4096 tokens x 7168 /
// 128-token top-8 dispatch): 16 lanes 17.3 / 5.7, 8 lanes 16.1 / 5.2,
// 4 lanes 16.6 / 5.3.
#ifndef WT_ACT_LANES
#define WT_ACT_LANES 8
#endif
constexpr int kActLanes = WT_ACT_LANES;
static_assert(kActLanes == 4 || kActLanes == 8 || kActLanes == 16, "lanes per block");

// Aligned path (cols, x_stride, q_stride multiples of 8, x 16-byte and q
// 8-byte aligned): L lanes per block, lane l owns the block's 16-byte chunks
// l, l + L, l + 2 L, ..., so that each load and store instruction covers
// consecutive bytes across the lanes of a wave.
template <int L>
__global__ void __launch_bounds__(kActThreads) act_quant_wide_kernel(ActArgs a) {
  constexpr int E = 128 / L;  // channels per lane
  constexpr int NC = E / 8;   // 16-byte chunks per lane
  constexpr int G = kActThreads / L;
  const uint32_t l = threadIdx.x & (L - 1);
  const uint32_t gblk = blockIdx.x * (uint32_t)G + threadIdx.x / L;
  uint32_t i = 0, b = 0;
  int64_t src = -1;
  if (gblk < a.n_blocks) {
    i = gblk / a.nb;
    b = gblk - i * a.nb;
    src = a.index ? (int64_t)ld_global<int32_t>(a.index + 4ull * i) : (int64_t)i;
  }
  const bool row_ok = src >= 0 && src < a.n_rows;
  const int64_t c0 = 128 * (int64_t)b + 8 * (int64_t)l;  // channel of the lane's first chunk
  const uint64_t xrow = a.x + 2ull * (uint64_t)(row_ok ? src : 0) * (uint64_t)a.x_stride;
  uint32_t w[NC][4];
#pragma unroll
  for (int ch = 0; ch < NC; ++ch) {
    w[ch][0] = w[ch][1] = w[ch][2] = w[ch][3] = 0u;
    if (row_ok && c0 + 8 * L * ch < a.cols) {
      const uint4 v = act_load16(xrow + 2ull * (uint64_t)(c0 + 8 * L * ch));
      w[ch][0] = v.x, w[ch][1] = v.y, w[ch][2] = v.z, w[ch][3] = v.w;
    }
  }
  uint32_t m = 0;
#pragma unroll
  for (int ch = 0; ch < NC; ++ch)
    m = pk_max_u16(m, pk_max_u16(pk_max_u16(abs2(w[ch][0]), abs2(w[ch][1])), pk_max_u16(abs2(w[ch][2]), abs2(w[ch][3]))));
  m = lanes_max<L>(max(m & 0xFFFFu, m >> 16));  // every lane of the group takes part
  if (!row_ok) return;
  const TileQ t = block_quant(m);
  const uint64_t qrow = a.q + (uint64_t)i * (uint64_t)a.q_stride;
#pragma unroll
  for (int ch = 0; ch < NC; ++ch)
    if (c0 + 8 * L * ch < a.cols) {
      const uint2 q = t.recip ? quant8<true>(w[ch], t) : quant8<false>(w[ch], t);
      act_store8(qrow + (uint64_t)(c0 + 8 * L * ch), q);
    }
  if (l == 0) st_global<float>(a.s + (uint64_t)i * (uint64_t)a.s_stride + 4ull * b, t.s);
}

}  // namespace

hipError_t launch_act_quant(const ActArgs &a, bool fast, hipStream_t stream) {
  if (a.n_blocks == 0) return hipSuccess;
  if (fast) {
    constexpr int G = kActThreads / kActLanes;
    const dim3 grid((a.n_blocks + G - 1) / G);
    hipLaunchKernelGGL((act_quant_wide_kernel<kActLanes>), grid, dim3(kActThreads), 0, stream, a);
  } else {
    const dim3 grid((a.n_blocks + kActGroups - 1) / kActGroups);
    hipLaunchKernelGGL(act_quant_kernel, grid, dim3(kActThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace wt
