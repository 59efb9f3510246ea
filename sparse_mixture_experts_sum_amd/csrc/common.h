// Internal helpers shared by the gfx950 kernels of the MoE library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
// Tokens per router workgroup; the per-block dispatch tables are indexed by it.
constexpr int kRouterTokens = 64;

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Order-preserving map of a float to uint32 (larger float -> larger key), with -0
// folded onto +0 so that the two zeros tie as they do in float comparison.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ float warp_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Block-wide exclusive scan of one integer (int or long long) per thread (blockDim.x a
// multiple of 64, at most 1024). `sh` must hold 17 of them. Returns the exclusive prefix;
// *total gets the sum over the block. All threads must call it.
template <class V>
__device__ inline V block_exclusive_scan(V v, V* sh, V* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  V incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    V u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  if (lane == 63) sh[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    V s = lane < nw ? sh[lane] : 0;
    V si = s;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      V u = __shfl_up(si, o);
      if (lane >= o) si += u;
    }
    if (lane < nw) sh[lane] = si - s;  // exclusive base of each wave
    if (lane == nw - 1) sh[16] = si;   // block total
  }
  __syncthreads();
  const V base = sh[wid];
  *total = sh[16];
  __syncthreads();  // sh may be reused by the caller right after
  return base + incl - v;
}

// Per-expert sums over the 64 tokens of a router block (kRouterTokens), in one fixed
// order shared by the router and the standalone statistics kernel, so that both give
// bitwise the same partials. 256 threads; thread tid holds v[i] for token tid / 4 of the
// block and expert (tid % 4) + 4 i, i < nper (zero for tokens past T). Order: an xor
// butterfly over the 16 tokens of each wave (the same tree in every lane), then the four
// wave sums in wave order. red: 4 x 64 floats of LDS. out[e] for e < E (E <= 64).
template <int NMAX>
__device__ __forceinline__ void block_expert_sums(float (&v)[NMAX], int nper, int E, float* red,
                                                  float* out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, part = tid & 3;
#pragma unroll
  for (int i = 0; i < NMAX; ++i) {
    if (i < nper) {
#pragma unroll
      for (int off = 4; off < 64; off <<= 1) v[i] += __shfl_xor(v[i], off);
      if ((lane >> 2) == 0 && part + 4 * i < E) red[wave * 64 + part + 4 * i] = v[i];
    }
  }
  __syncthreads();
  if (tid < E) out[tid] = ((red[tid] + red[64 + tid]) + red[128 + tid]) + red[192 + tid];
}

// Load-balancing statistics from per-block partials (Mixture of Experts（MoE）の理論と実装,
// load_balancing_loss; the Korean page's compute_load_balancing_loss and router_z_loss):
//   f[e] = cnt[e] / T, p[e] = (sum over blocks of blk_psum[b, e]) / T,
//   loss = E * sum_e (f[e] / k) * p[e], z_loss = (sum over blocks of blk_zsum[b]) / T.
// One fixed order whichever kernel calls it: item i (expert i < E, the z-loss for i = E)
// belongs to wave i % (waves of the block), whose lane l adds blocks l, l + 64, ... in
// double, then an xor tree over the lanes; thread 0 adds the loss terms in expert order.
// The bits of every item depend only on the lane it is summed in, so blocks of any number
// of waves give the same results. A wave takes IPR of its items at a time: eight loads per
// lane and item in flight (the partials were just written by other CUs, so each load waits
// for memory), then each item's values added in block order; IPR changes no bit, only the
// registers it takes (4 for the 256-thread dispatch, 1 where 1024 threads leave 128
// registers each). cnt: the E assignment totals, in LDS, visible to all threads. A multiple
// of 64 threads, at least 128; every thread must call it. Null outputs are skipped.
template <int IPR>
__device__ __forceinline__ void aux_stats_block(const int* cnt, const float* __restrict__ blk_psum,
                                                const float* __restrict__ blk_zsum, int nblk,
                                                int T, int E, int k, float* f, float* p,
                                                float* loss, float* z_loss) {
  __shared__ double item[65];
  __shared__ double term[64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  for (int i0 = wave; i0 <= E; i0 += nwaves * IPR) {
    double v[IPR];
    const float* src[IPR];
    size_t stride[IPR];
#pragma unroll
    for (int r = 0; r < IPR; ++r) {
      const int i = i0 + r * nwaves;
      v[r] = 0.0;
      src[r] = i > E ? nullptr : (i < E ? (blk_psum ? blk_psum + i : nullptr) : blk_zsum);
      stride[r] = i < E ? (size_t)E : 1;
    }
    for (int b0 = lane; b0 < nblk; b0 += 64 * 8) {
      float x8[IPR][8];
#pragma unroll
      for (int r = 0; r < IPR; ++r)
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int b = b0 + 64 * u;
          x8[r][u] = (src[r] && b < nblk) ? src[r][(size_t)b * stride[r]] : 0.f;
        }
#pragma unroll
      for (int r = 0; r < IPR; ++r)
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (src[r] && b0 + 64 * u < nblk) v[r] += (double)x8[r][u];
    }
#pragma unroll
    for (int r = 0; r < IPR; ++r) {
      const int i = i0 + r * nwaves;
      if (i > E) continue;  // (uniform over the wave)
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) v[r] += __shfl_xor(v[r], o);
      if (lane == 0) item[i] = v[r];
    }
  }
  __syncthreads();
  if (threadIdx.x == 64 && z_loss && blk_zsum) *z_loss = (float)(item[E] / (double)T);
  if (threadIdx.x < E) {
    const int e = threadIdx.x;
    const float fe = (float)((double)cnt[e] / (double)T);
    const float pe = (float)(item[e] / (double)T);
    if (f) f[e] = fe;
    if (p) p[e] = pe;
    term[e] = ((double)fe / (double)k) * (double)pe;
  }
  __syncthreads();
  if (threadIdx.x == 0 && loss) {
    double sacc = 0.0;
    for (int i = 0; i < E; ++i) sacc += term[i];
    *loss = (float)((double)E * sacc);
  }
}
