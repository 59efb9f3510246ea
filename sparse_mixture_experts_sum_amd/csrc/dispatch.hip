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
    aux_stats_block<1>(cnt_sh, a.blk_psum, a.blk_zsum, nblk, a.T, E, a.k, a.f, a.p, a.loss, a.z_loss);
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

// ---------------------------------------------------------------------------------
// Token choice in one kernel, for up to kFusedMaxBlocks router blocks: the prefix sums of
// the dispatch scan and the permutation above, with no launch between them. Block b takes
// router block b's tokens: it sums every expert's per-block counts itself (the totals, and
// the part from blocks before b), derives the clamped group starts, and writes its slots'
// rows (and, where rows are copied, the rows). Block nblk, when statistics are requested,
// reduces f, p, loss and z_loss from the totals and the router's per-block partials in the
// fixed order of aux_stats_block (the same bits as the standalone statistics). The counts
// are re-read by every block (E * nblk ints each), which is why larger batches take the
// two-kernel path.
// ---------------------------------------------------------------------------------
// NT threads per block: 256 (four waves take 16 experts' counts per round) up to 16 experts,
// 1024 beyond, so that all 64 experts' counts come in one round and the statistics block
// has 16 waves (64 experts: 29.7 -> 16.2 us; with 8 experts the larger blocks cost 2 us).
template <int EB, int NT>
__global__ __launch_bounds__(NT) void dispatch_tc_kernel(DispatchArgs a) {
  constexpr int kDispatchWaves = NT / 64;
  __shared__ int pre_sh[64];   // this block's slots of expert e come after pre_sh[e] others
  __shared__ int tot_sh[64];   // assignments per expert (before any capacity)
  __shared__ int gs_sh[64];    // group start of expert e (clamped sizes)
  __shared__ int pos_sh[kRouterTokens * 8];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nblk = a.nblk, E = a.E, k = a.k, T = a.T;
  // wave w sums experts w, w + waves, ...: four experts' rows at a time (16 per round at 256
  // threads, all 64 at 1024), every load of the four issued before any is added (up to 32 in
  // flight per lane), then a wave reduction each
  constexpr int EPC = 4, LPR = kFusedMaxBlocks / 64;  // experts per round, loads per row
  for (int e0 = wave; e0 < E; e0 += kDispatchWaves * EPC) {
    int c[EPC][LPR];
#pragma unroll
    for (int i = 0; i < EPC; ++i) {
      const int e = e0 + kDispatchWaves * i;
      const int32_t* row = a.blk_counts + (size_t)min(e, E - 1) * nblk;
#pragma unroll
      for (int j = 0; j < LPR; ++j) {
        const int jb = lane + 64 * j;
        c[i][j] = (e < E && jb < nblk) ? row[jb] : 0;
      }
    }
#pragma unroll
    for (int i = 0; i < EPC; ++i) {
      int pre = 0, tot = 0;
#pragma unroll
      for (int j = 0; j < LPR; ++j) {
        tot += c[i][j];
        pre += lane + 64 * j < b ? c[i][j] : 0;
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        pre += __shfl_xor(pre, o);
        tot += __shfl_xor(tot, o);
      }
      const int e = e0 + kDispatchWaves * i;
      if (lane == 0 && e < E) {
        pre_sh[e] = pre;
        tot_sh[e] = tot;
      }
    }
  }
  __syncthreads();
  if (b == nblk) {  // the statistics block
    // (items per round: 4 in 64 registers per lane at 256 threads, 2 within 1024 threads' 128)
    aux_stats_block<NT == 1024 ? 2 : 4>(tot_sh, a.blk_psum, a.blk_zsum, nblk, T, E, k, a.f, a.p,
                                        a.loss, a.z_loss);
    return;
  }
  if (wave == 0) {  // clamped sizes and their exclusive prefix (E <= 64)
    const int c = lane < E ? tot_sh[lane] : 0;
    const int cc = min(c, a.cap);
    int incl = cc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o);
      if (lane >= o) incl += u;
    }
    if (lane < E) gs_sh[lane] = incl - cc;
    if (b == 0) {
      if (lane < E) {
        a.offsets[lane] = incl - cc;
        a.counts[lane] = c;
        if (a.user_counts) a.user_counts[lane] = c;
      }
      if (lane == E - 1) a.offsets[E] = incl;
    }
  }
  if (b == 0 && a.sk_flags)
    for (int i = tid; i < kStreamKSlots; i += blockDim.x) a.sk_flags[i] = 0;
  __syncthreads();
  // slots: row = group start + earlier blocks' slots of the expert + rank in this block
  const int t0 = b * kRouterTokens, ntok = min(kRouterTokens, T - t0);
  const int R = T * k;
  for (int q = tid; q < ntok * k; q += blockDim.x) {
    const size_t sidx = (size_t)t0 * k + q;
    const int e = a.idx[sidx];
    const int rank = pre_sh[e] + a.lrank[sidx];  // among the expert's slots, token order
    int p = rank >= a.cap ? -1 : gs_sh[e] + rank;  // dropped by the capacity
    if (p >= R) p = -1;  // unreachable for consistent tables; never write outside
    a.pos[sidx] = p;
    pos_sh[q] = p;
    if (p >= 0) a.src[p] = t0 + q / k;
  }
  if (a.cap != INT_MAX || a.x_perm) __syncthreads();
  if (a.cap != INT_MAX && tid < ntok) {
    // a token that lost a slot: its kept weights divided by their sum, added in slot order
    const size_t s0 = (size_t)(t0 + tid) * k;
    bool lost = false;
    float sk = 0.f;
    for (int j = 0; j < k; ++j) {
      const bool kept = pos_sh[tid * k + j] >= 0;
      lost |= !kept;
      if (kept) sk += a.w[s0 + j];
    }
    if (lost) {
      for (int j = 0; j < k; ++j) {
        const float wj = a.w[s0 + j];
        const float wk = a.renorm ? (sk > 0.f ? wj / sk : 0.f) : wj;
        a.w[s0 + j] = pos_sh[tid * k + j] >= 0 ? wk : 0.f;
      }
    }
  }
  if (!a.x_perm) return;
  // row copies: one wave per token, 16-byte pieces, to each kept slot's row
  const size_t row_bytes = (size_t)a.d * EB;
  const int nch = (int)(row_bytes / 16);
  for (int tt = wave; tt < ntok; tt += kDispatchWaves) {
    const char* xr = a.x + (size_t)(t0 + tt) * row_bytes;
    for (int c = lane; c < nch; c += 64) {
      const u32x4 v = ld16(xr + 16 * (size_t)c);
      for (int j = 0; j < k; ++j) {
        const int pj = pos_sh[tt * k + j];
        if (pj >= 0) st16(a.x_perm + (size_t)pj * row_bytes + 16 * (size_t)c, v);
      }
    }
  }
}

}  // namespace

hipError_t launch_dispatch_tc(const DispatchArgs& a, hipStream_t s) {
  if (a.E < 1 || a.E > 64 || a.k < 1 || a.k > 8 || a.nblk > kFusedMaxBlocks)
    return hipErrorInvalidValue;
  const bool stats = a.f || a.p || a.loss || a.z_loss;
  dim3 grid(a.nblk + (stats ? 1 : 0));
  if (a.E > 16) {
    if (a.elt_bytes == 2)
      dispatch_tc_kernel<2, 1024><<<grid, 1024, 0, s>>>(a);
    else
      dispatch_tc_kernel<4, 1024><<<grid, 1024, 0, s>>>(a);
  } else {
    if (a.elt_bytes == 2)
      dispatch_tc_kernel<2, 256><<<grid, 256, 0, s>>>(a);
    else
      dispatch_tc_kernel<4, 256><<<grid, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

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
