// Dispatch: prefix sum over the router's per-block expert histogram and the stable
// permutation of token rows into expert-contiguous order.
//
// The expert-parallel dispatch of "Sparse Mixture of Experts(MoE) 아키텍처 심층 분석"
// (ExpertParallelRouter.dispatch) counts tokens per destination and sorts the token
// rows by expert before sending them; here the same grouping feeds the grouped GEMMs
// of one GPU. Row order inside an expert's group is the flattened (token, slot)
// order, so the permutation is stable and deterministic without atomics.
#include <limits.h>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int kScanThreads = 1024;

// One workgroup. Entry q = e*nblk + b of the per-block counts (expert-major, [E, nblk])
// holds block b's slots for expert e; its exclusive prefix is the first slot of block b's
// slots for expert e in the expert's flattened (token, slot) order, and the prefix at
// (e, 0) is the start of expert e's group. With an expert capacity `cap`, expert e keeps
// only the first cap of its slots: its group shrinks to min(count, cap) rows, the groups
// are laid out from those sizes, and base[b, e] is the clamped group start plus the
// block's unclamped prefix (rows at or past start + cap are dropped by the permute).
// counts stay the unclamped assignments. cap = INT_MAX: no capacity.
// When any of f, p, loss, z_loss is given, the load-balancing statistics follow from the
// same totals (aux_stats_block: the order of the standalone statistics kernel).
constexpr int kScanCache = 16;  // entries per thread kept in registers between the passes
__global__ __launch_bounds__(kScanThreads) void dispatch_scan_kernel(ScanArgs a) {
  __shared__ int sh[17];
  __shared__ int off_sh[65];   // unclamped group starts
  __shared__ int offc_sh[65];  // group starts from the clamped sizes
  __shared__ int cnt_sh[64];
  const int nblk = a.nblk, E = a.E;
  const long n = (long)nblk * E;
  const int tid = threadIdx.x;
  const long per = (n + kScanThreads - 1) / kScanThreads;
  const long qb = min(n, (long)tid * per), qe = min(n, qb + per);
  const bool cached = per <= kScanCache;
  int v[kScanCache];
  int local = 0;
  if (cached) {
#pragma unroll
    for (int i = 0; i < kScanCache; ++i) {
      v[i] = qb + i < qe ? a.blk_counts[qb + i] : 0;
      local += v[i];
    }
  } else {
    for (long q = qb; q < qe; ++q) local += a.blk_counts[q];
  }
  int total;
  const int run0 = block_exclusive_scan(local, sh, &total);
  int run = run0;
  if (cached) {
#pragma unroll
    for (int i = 0; i < kScanCache; ++i) {
      const long q = qb + i;
      if (q < qe && q % nblk == 0) off_sh[q / nblk] = run;
      run += v[i];
    }
  } else {
    for (long q = qb; q < qe; ++q) {
      if (q % nblk == 0) off_sh[q / nblk] = run;
      run += a.blk_counts[q];
    }
  }
  if (tid == 0) off_sh[E] = total;
  __syncthreads();
  if (tid < 64) {  // wave 0: clamped sizes and their exclusive prefix (E <= 64)
    const int c = tid < E ? off_sh[tid + 1] - off_sh[tid] : 0;
    cnt_sh[tid] = c;
    const int cc = min(c, a.cap);
    int incl = cc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o);
      if (tid >= o) incl += u;
    }
    if (tid < E) offc_sh[tid] = incl - cc;
    if (tid == E - 1) offc_sh[E] = incl;
  }
  __syncthreads();
  run = run0;
  if (cached) {
#pragma unroll
    for (int i = 0; i < kScanCache; ++i) {
      const long q = qb + i;
      if (q < qe) {
        const int e = (int)(q / nblk), b = (int)(q - (long)e * nblk);
        a.base[(size_t)b * E + e] = offc_sh[e] + (run - off_sh[e]);
      }
      run += v[i];
    }
  } else {
    for (long q = qb; q < qe; ++q) {
      const int e = (int)(q / nblk), b = (int)(q - (long)e * nblk);
      a.base[(size_t)b * E + e] = offc_sh[e] + (run - off_sh[e]);
      run += a.blk_counts[q];
    }
  }
  if (tid <= E) a.offsets[tid] = offc_sh[tid];
  if (tid < E) {
    a.counts[tid] = cnt_sh[tid];
    if (a.user_counts) a.user_counts[tid] = cnt_sh[tid];
  }
  if (a.f || a.p || a.loss || a.z_loss)
    aux_stats_block(cnt_sh, a.blk_psum, a.blk_zsum, nblk, a.T, E, a.k, a.f, a.p, a.loss, a.z_loss);
}

// One wave per token: slots first (pos, src), then the row copy to every slot's row.
// With an expert capacity (cap < INT_MAX) a slot whose rank among its expert's slots
// (flattened token order) is cap or more is dropped: pos = -1, weight 0, and when the
// token lost a slot its kept weights are divided by their sum (renorm) — the capacity
// routing of 机器学习基础系列——混合专家模型 (expert_capacity_routing). x_perm == nullptr:
// slots and weights only (bf16 layers, whose gate/up GEMM gathers the rows through src,
// and routing without the layer).
template <int EB>
__global__ __launch_bounds__(256) void permute_tc_kernel(const char* __restrict__ x, int T, int d,
                                                         int E, int k, const int32_t* __restrict__ idx,
                                                         const int32_t* __restrict__ lrank,
                                                         const int32_t* __restrict__ base,
                                                         const int32_t* __restrict__ offsets,
                                                         int cap, int renorm, int32_t* pos,
                                                         int32_t* src, float* w,
                                                         char* __restrict__ x_perm,
                                                         int32_t* sk_flags) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (sk_flags && blockIdx.x == 0)
    for (int i = threadIdx.x; i < kStreamKSlots; i += blockDim.x) sk_flags[i] = 0;
  if (t >= T) return;
  const int R = T * k;
  int p = -1;
  if (lane < k) {
    const int e = idx[(size_t)t * k + lane];
    p = base[(size_t)(t / kRouterTokens) * E + e] + lrank[(size_t)t * k + lane];
    if (p - offsets[e] >= cap) p = -1;  // dropped by the capacity
    if (p < 0 || p >= R) p = -1;  // unreachable for consistent tables; never write outside
    pos[(size_t)t * k + lane] = p;
    if (p >= 0) src[p] = t;
  }
  if (cap != INT_MAX) {
    const uint64_t slots = __ballot(lane < k), kept = __ballot(lane < k && p >= 0);
    if (kept != slots) {  // the token lost a slot (uniform over the wave)
      const float wj = lane < k ? w[(size_t)t * k + lane] : 0.f;
      float sk = p >= 0 ? wj : 0.f;
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) sk += __shfl_xor(sk, o);  // lanes 0..7, fixed tree
      if (lane < k) {
        const float wk = renorm ? (sk > 0.f ? wj / sk : 0.f) : wj;
        w[(size_t)t * k + lane] = p >= 0 ? wk : 0.f;
      }
    }
  }
  if (!x_perm) return;
  const size_t row_bytes = (size_t)d * EB;
  const int nch = (int)(row_bytes / 16);
  const char* xr = x + (size_t)t * row_bytes;
  for (int c0 = 0; c0 < nch; c0 += 64 * 4) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + u * 64 + lane;
      if (c < nch) v[u] = ld16(xr + 16 * (size_t)c);
    }
    for (int j = 0; j < k; ++j) {
      const int pj = __shfl(p, j);
      if (pj < 0) continue;
      char* dst = x_perm + (size_t)pj * row_bytes;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + u * 64 + lane;
        if (c < nch) st16(dst + 16 * (size_t)c, v[u]);
      }
    }
  }
}

// One wave per routed row of expert choice: row e*C + c takes token idx[e, c].
__global__ __launch_bounds__(256) void permute_ec_kernel(const char* __restrict__ x, size_t row_bytes,
                                                         int R, const int32_t* __restrict__ idx,
                                                         int32_t* src, char* __restrict__ x_perm,
                                                         int32_t* sk_flags) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (sk_flags && blockIdx.x == 0)
    for (int i = threadIdx.x; i < kStreamKSlots; i += blockDim.x) sk_flags[i] = 0;
  if (r >= R) return;
  const int t = idx[r];
  if (lane == 0) src[r] = t;
  if (!x_perm) return;
  const int nch = (int)(row_bytes / 16);
  const char* xr = x + (size_t)t * row_bytes;
  char* dst = x_perm + (size_t)r * row_bytes;
  for (int c = lane; c < nch; c += 64) st16(dst + 16 * (size_t)c, ld16(xr + 16 * (size_t)c));
}

}  // namespace

hipError_t launch_dispatch_scan(const ScanArgs& a, hipStream_t s) {
  if (a.E < 1 || a.E > 64) return hipErrorInvalidValue;
  dispatch_scan_kernel<<<1, kScanThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_permute_tc(const void* x, int elt_bytes, int T, int d, int E, int k,
                             const int32_t* idx, const int32_t* lrank, const int32_t* base,
                             const int32_t* offsets, int cap, int renorm, int32_t* pos,
                             int32_t* src, float* w, void* x_perm, int32_t* sk_flags,
                             hipStream_t s) {
  dim3 grid((T + 3) / 4), block(256);
  if (elt_bytes == 2)
    permute_tc_kernel<2><<<grid, block, 0, s>>>(static_cast<const char*>(x), T, d, E, k, idx, lrank,
                                                base, offsets, cap, renorm, pos, src, w,
                                                static_cast<char*>(x_perm), sk_flags);
  else
    permute_tc_kernel<4><<<grid, block, 0, s>>>(static_cast<const char*>(x), T, d, E, k, idx, lrank,
                                                base, offsets, cap, renorm, pos, src, w,
                                                static_cast<char*>(x_perm), sk_flags);
  return hipGetLastError();
}

hipError_t launch_permute_ec(const void* x, int elt_bytes, int d, int E, int C,
                             const int32_t* idx, int32_t* src, void* x_perm, int32_t* sk_flags,
                             hipStream_t s) {
  const int R = E * C;
  dim3 grid((R + 3) / 4), block(256);
  permute_ec_kernel<<<grid, block, 0, s>>>(static_cast<const char*>(x), (size_t)d * elt_bytes, R, idx,
                                           src, static_cast<char*>(x_perm), sk_flags);
  return hipGetLastError();
}
