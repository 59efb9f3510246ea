// Weighted un-permute and combine, and the load-balancing statistics.
//
// Combine: y_t = sum over the token's experts of weight * E_e(x_t) (qiita primer,
// fourth router equation; "Mixture of Experts（MoE）の理論と実装", MoELayer.forward).
// Expert outputs o sit in expert-contiguous rows; token t reads its k rows through
// pos[t, :] and sums them in slot order in fp32, so the result does not depend on
// scheduling. Expert choice (the Korean page's ExpertChoiceGating dispatch mask):
// token t takes, per expert, the row the expert gave it (if any) from the expert's
// ascending token list, and sums the chosen rows in ascending expert order.
//
// Statistics ("Mixture of Experts（MoE）の理論と実装", load_balancing_loss; the Korean
// page's compute_load_balancing_loss): f_e = count_e / T, p_e = mean_t probs[t, e],
// loss = E * sum_e (f_e / k) * p_e, from per-block partials in a fixed order.
#include "common.h"
#include "kernels.h"

namespace {

// one wave per token, 4 tokens per workgroup; k <= 8
__global__ __launch_bounds__(256) void combine_tc_kernel(const float* __restrict__ o,
                                                         const int32_t* __restrict__ pos,
                                                         const float* __restrict__ w, int T, int d,
                                                         int k, float* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int pj = 0;
  float wj = 0.f;
  if (lane < k) {
    pj = pos[(size_t)t * k + lane];
    wj = w[(size_t)t * k + lane];
  }
  int prow[8];
  float pw[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    prow[j] = __shfl(pj, j);
    pw[j] = __shfl(wj, j);
  }
  const int nch = d / 4;
  float* yr = y + (size_t)t * d;
  // four 16-byte chunks per lane and slot in flight at once; o is read and y written
  // once, so both bypass the caches' retention (non-temporal), which leaves the
  // last-level cache to the data the next kernels reuse
  int c = lane;
  for (; c + 192 < nch; c += 256) {
    f32x4 v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v[u][j] = (j < k && prow[j] >= 0)
                      ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(
                            o + (size_t)prow[j] * d + 4 * (c + 64 * u)))
                      : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < k) acc += pw[j] * v[u][j];
      __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(yr + 4 * (c + 64 * u)));
    }
  }
  for (; c < nch; c += 64) {
    f32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j] = (j < k && prow[j] >= 0)
                 ? __builtin_nontemporal_load(
                       reinterpret_cast<const f32x4*>(o + (size_t)prow[j] * d + 4 * c))
                 : f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < k) acc += pw[j] * v[j];
    __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(yr + 4 * c));
  }
}

// one wave per token; lane e < E searches expert e's token list
__global__ __launch_bounds__(256) void combine_ec_kernel(const float* __restrict__ o,
                                                         const int32_t* __restrict__ idx,
                                                         const float* __restrict__ score, int T,
                                                         int d, int E, int C,
                                                         float* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int row = -1;
  float sc = 0.f;
  if (lane < E) {
    const int32_t* list = idx + (size_t)lane * C;
    int lo = 0, hi = C;  // first position with list[pos] >= t
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (list[mid] < t) lo = mid + 1;
      else hi = mid;
    }
    if (lo < C && list[lo] == t) {
      row = lane * C + lo;
      sc = score[(size_t)lane * C + lo];
    }
  }
  const uint64_t found = __ballot(row >= 0);
  const int nch = d / 4;
  float* yr = y + (size_t)t * d;
  // every lane runs every round (chunks c0 + lane, the lanes past the row's end idle), so
  // that the shuffles read their source lanes while those are active: a shuffle from a
  // lane outside the exec mask reads nothing (d_model < 256 leaves lanes d_model / 4 and
  // up without a chunk, and expert e's row and score sit in lane e)
  for (int c0 = 0; c0 < nch; c0 += 64) {
    const int c = c0 + lane;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    uint64_t m = found;
    while (m) {
      const int e = __ffsll((unsigned long long)m) - 1;
      m &= m - 1;
      const int r = __shfl(row, e);
      const float s = __shfl(sc, e);
      if (c < nch) {
        const f32x4 v = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(o + (size_t)r * d + 4 * c));
        acc += s * v;
      }
    }
    if (c < nch) __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(yr + 4 * c));
  }
}

// Expert choice, a workgroup per block of kEcCombineTokens consecutive tokens (d_model >= 512).
// The experts' token lists are ascending, so the block's entries in expert e's list are one
// run, whose ends the select kernel wrote into the run table (runs[e][b], runs[e][b + 1]): no
// search. The entries are laid out by (token, expert), and every thread walks that list for
// its 16-byte column chunks: per token, acc = 0, then acc += score * o[row] in ascending expert
// order (the same operations, in the same order, as combine_ec_kernel), eight rows' loads
// issued before they are added. Tokens no expert took get zeros.
constexpr int kEcTok = kEcCombineTokens;

__global__ __launch_bounds__(256) void combine_ec_block_kernel(const float* __restrict__ o,
                                                               const int32_t* __restrict__ idx,
                                                               const float* __restrict__ score,
                                                               const int32_t* __restrict__ runs,
                                                               int T, int d, int E, int C,
                                                               float* __restrict__ y) {
  __shared__ int run_lo[64], run_hi[64];
  __shared__ int tab[kEcTok][64];       // row of (token, expert), or -1
  __shared__ int ftok[kEcTok * 64];     // the block's entries in (token, expert) order
  __shared__ int frow[kEcTok * 64];
  __shared__ float fsc[kEcTok * 64];
  __shared__ int empty_tok[kEcTok];
  __shared__ int nflat;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kEcTok;
  const int ntok = min(kEcTok, T - t0);

  // 1. each expert's run of entries in [t0, t0 + ntok), from the select's run table
  if (tid < E) {
    const int32_t* r = runs + (size_t)tid * ec_run_stride(T) + blockIdx.x;
    run_lo[tid] = r[0];
    run_hi[tid] = r[1];
  }
  for (int i = tid; i < kEcTok * 64; i += 256) tab[i >> 6][i & 63] = -1;
  __syncthreads();
  // 2. the (token, expert) table: at most ntok entries per expert
  for (int i = tid; i < E * kEcTok; i += 256) {
    const int e = i / kEcTok, j = run_lo[e] + i % kEcTok;
    if (j < run_hi[e]) {
      const int tl = idx[(size_t)e * C + j] - t0;  // in [0, ntok) by the run table
      if (tl >= 0 && tl < ntok) tab[tl][e] = e * C + j;
    }
  }
  __syncthreads();
  // 3. wave 0 compacts the table in (token, expert) order; wave 1 marks the empty tokens
  if (wave == 0) {
    int base = 0;
    const int n = ntok * E;
    for (int i0 = 0; i0 < n; i0 += 64) {
      const int i = i0 + lane;
      const int tl = i / E, e = i - tl * E;
      const int r = i < n ? tab[tl][e] : -1;
      const uint64_t m = __ballot(r >= 0);
      if (r >= 0) {
        const int at = base + __popcll(m & ((1ull << lane) - 1ull));
        ftok[at] = tl;
        frow[at] = r;
        fsc[at] = score[r];
      }
      base += __popcll(m);
    }
    if (lane == 0) nflat = base;
  } else if (wave == 1 && lane < ntok) {
    int any = 0;
    for (int e = 0; e < E; ++e) any |= tab[lane][e] >= 0;
    empty_tok[lane] = !any;
  }
  __syncthreads();
  const int n = nflat, nch = d / 4;
  for (int c = tid; c < nch; c += 256) {
    for (int tl = 0; tl < ntok; ++tl)
      if (empty_tok[tl])
        __builtin_nontemporal_store(f32x4{0.f, 0.f, 0.f, 0.f},
                                    reinterpret_cast<f32x4*>(y + (size_t)(t0 + tl) * d + 4 * c));
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    int cur = -1;
    for (int j0 = 0; j0 < n; j0 += 8) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = j0 + u < n ? __builtin_nontemporal_load(
                                reinterpret_cast<const f32x4*>(o + (size_t)frow[j0 + u] * d + 4 * c))
                          : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (j0 + u >= n) break;
        const int tl = ftok[j0 + u];
        if (tl != cur) {
          if (cur >= 0)
            __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(y + (size_t)(t0 + cur) * d + 4 * c));
          acc = f32x4{0.f, 0.f, 0.f, 0.f};
          cur = tl;
        }
        const float sc = fsc[j0 + u];
        acc += sc * v[u];
      }
    }
    if (cur >= 0)
      __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(y + (size_t)(t0 + cur) * d + 4 * c));
  }
}

// per block of kRouterTokens tokens: slot counts per expert and probability sums
__global__ __launch_bounds__(256) void aux_partials_kernel(const float* __restrict__ probs,
                                                           const int32_t* __restrict__ idx, int T,
                                                           int E, int k, int32_t* blk_counts,
                                                           float* blk_psum) {
  __shared__ int cnt[64];
  __shared__ float red[256];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kRouterTokens;
  const int ntok = min(kRouterTokens, T - t0);
  if (tid < 64) cnt[tid] = 0;
  __syncthreads();
  for (int q = tid; q < ntok * k; q += 256) {
    const int e = idx[(size_t)t0 * k + q];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  // the router's block sums, in the router's order (block_expert_sums)
  const int tok = tid >> 2, part = tid & 3;
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = part + 4 * i;
    v[i] = (tok < ntok && e < E) ? probs[(size_t)(t0 + tok) * E + e] : 0.f;
  }
  block_expert_sums<16>(v, (E + 3) / 4, E, red, blk_psum + (size_t)blockIdx.x * E);
  __syncthreads();
  if (tid < E) blk_counts[(size_t)tid * gridDim.x + blockIdx.x] = cnt[tid];
}

// 1024 threads: assignment totals per expert from the per-block counts ([E, nblk],
// expert-major), then the statistics in the shared fixed order (aux_stats_block).
__global__ __launch_bounds__(1024) void aux_final_kernel(const int32_t* __restrict__ blk_counts,
                                                         const float* __restrict__ blk_psum, int nblk,
                                                         int T, int E, int k, float* f, float* p,
                                                         float* loss, int32_t* counts,
                                                         const float* __restrict__ blk_zsum,
                                                         float* z_loss) {
  __shared__ int cnt[64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // wave w totals experts w, w + 16, ...: a lane-strided sum, then an xor tree
  for (int e = wave; e < E; e += 16) {
    int c = 0;
    for (int b = lane; b < nblk; b += 64) c += blk_counts[(size_t)e * nblk + b];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) c += __shfl_xor(c, o);
    if (lane == 0) cnt[e] = c;
  }
  __syncthreads();
  if (counts && threadIdx.x < E) counts[threadIdx.x] = cnt[threadIdx.x];
  aux_stats_block<1>(cnt, blk_psum, blk_zsum, nblk, T, E, k, f, p, loss, z_loss);
}

__global__ void fill_zero_kernel(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

}  // namespace

hipError_t launch_combine_tc(const float* o, const int32_t* pos, const float* w, int T, int d,
                             int k, float* y, hipStream_t s) {
  combine_tc_kernel<<<(T + 3) / 4, 256, 0, s>>>(o, pos, w, T, d, k, y);
  return hipGetLastError();
}

hipError_t launch_combine_ec(const float* o, const int32_t* idx, const float* score,
                             const int32_t* runs, int T, int d, int E, int C, float* y,
                             hipStream_t s) {
  // (narrower rows leave most of a block's threads without a column chunk)
  if (runs && d >= 512)
    combine_ec_block_kernel<<<ec_run_stride(T) - 1, 256, 0, s>>>(o, idx, score, runs, T, d, E, C,
                                                                 y);
  else
    combine_ec_kernel<<<(T + 3) / 4, 256, 0, s>>>(o, idx, score, T, d, E, C, y);
  return hipGetLastError();
}

hipError_t launch_aux_partials(const float* probs, const int32_t* idx, int T, int E, int k,
                               int32_t* blk_counts, float* blk_psum, hipStream_t s) {
  const int nblk = (T + kRouterTokens - 1) / kRouterTokens;
  aux_partials_kernel<<<nblk, 256, 0, s>>>(probs, idx, T, E, k, blk_counts, blk_psum);
  return hipGetLastError();
}

hipError_t launch_aux_final(const int32_t* blk_counts, const float* blk_psum, int nblk, int T,
                            int E, int k, float* f, float* p, float* loss, int32_t* counts,
                            const float* blk_zsum, float* z_loss, hipStream_t s) {
  aux_final_kernel<<<1, 1024, 0, s>>>(blk_counts, blk_psum, nblk, T, E, k, f, p, loss, counts,
                                      blk_zsum, z_loss);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  const int grid = (int)min((size_t)1024, (n + 255) / 256);
  fill_zero_kernel<<<grid, 256, 0, s>>>(static_cast<uint32_t*>(ptr), n);
  return hipGetLastError();
}
