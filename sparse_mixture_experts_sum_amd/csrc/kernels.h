// Launch wrappers for the gfx950 kernels (internal; the public ABI is include/moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

struct RouterArgs {
  const void* x;        // [T, d] dtype
  const void* Wg;       // [d, E] dtype
  const float* bias;    // [E] or nullptr
  // token choice, optional training noise: logits + softplus(x Wn) * eps, or + eps
  // when Wn is nullptr; eps from the eps array, or drawn in the kernel (draw = 1: the
  // counter-based normal draw of (seed, offset) times noise_scale); none when eps is
  // nullptr and draw is 0
  const void* Wn;       // [d, E] dtype or nullptr
  const float* eps;     // [T, E] or nullptr
  int draw;
  uint32_t seed_lo, seed_hi, off_lo, off_hi;
  float noise_scale;
  int T, d, E, k, renorm;
  // token choice outputs
  int32_t* idx;         // [T, k]
  float* w;             // [T, k]
  float* probs;         // [T, E] or nullptr
  int32_t* lrank;       // [T, k] rank of the slot among equal experts within its block
  int32_t* blk_counts;  // [E, nblk] (expert-major)
  float* blk_psum;      // [nblk, E] column sums of probs over the block's tokens
  // both modes, optional: per block, sum over its tokens of logsumexp(logits)^2
  float* blk_zsum;      // [nblk] or nullptr
  // expert choice output
  float* logitsT;       // [E, T] (expert choice only)
};

// Token-choice router (logits, softmax, top-k, weights, per-block histogram and
// slot ranks, per-block probability sums) or, with ec = 1, expert-choice logits; in
// either mode, when blk_zsum is set, the per-block z-loss partials.
hipError_t launch_router(const RouterArgs& a, int bf16, int ec, hipStream_t s);

// Tokens per workgroup of the expert-choice combine, and the granularity of the run table
// the select writes for it.
constexpr int kEcCombineTokens = 16;
// Entries per expert of that table: one per block of kEcCombineTokens tokens, plus the end.
__host__ __device__ inline int ec_run_stride(int T) {
  return T / kEcCombineTokens + (T % kEcCombineTokens != 0) + 1;  // (no T + 15: T may be 2^31 - 1)
}

// Expert choice: per expert, softmax over tokens, top-C tokens (ascending token
// order) and scores. Also writes offsets[e] = e*C for e <= E, counts (optional),
// src (optional: the token of each row e*C + c, the same list as idx, for the gate/up
// GEMM's gather), clears the stream-K flags (optional), and (optional) the run table
// runs [E, ec_run_stride(T)]: runs[e][b] = entries of expert e's list with token below
// b * kEcCombineTokens (the last entry, C).
hipError_t launch_ec_select(const float* logitsT, int T, int E, int C, int32_t* idx, float* score,
                            float* probs, int32_t* offsets, int32_t* counts, int32_t* src,
                            int32_t* sk_flags, int32_t* runs, hipStream_t s);

// Dispatch prefix sum over per-block counts blk_counts [E, nblk] (expert-major):
// counts[E] (unclamped), offsets[E+1] (group starts; with an expert capacity cap the
// groups hold min(count, cap) rows), base[nblk, E] (row of each (block, expert) pair's
// first slot), optional user counts; cap = INT_MAX: no capacity. Optionally also the
// load-balancing statistics f, p, loss and z_loss from the per-block partials, in the
// same order as launch_aux_final.
struct ScanArgs {
  const int32_t* blk_counts;  // [E, nblk]
  int nblk, E, cap;
  int32_t* counts;            // [E]
  int32_t* offsets;           // [E+1]
  int32_t* base;              // [nblk, E]
  int32_t* user_counts;       // [E] or nullptr
  // statistics (all optional)
  const float* blk_psum;      // [nblk, E]
  const float* blk_zsum;      // [nblk]
  int T, k;
  float *f, *p, *loss, *z_loss;
};
hipError_t launch_dispatch_scan(const ScanArgs& a, hipStream_t s);

// Token choice, the scan and the permutation in one launch (up to kFusedMaxBlocks router
// blocks): offsets, counts, pos, src, capacity drops and renormalised weights, row copies
// when x_perm is set, and (with any of f, p, loss, z_loss) the statistics, all as from
// launch_dispatch_scan followed by launch_permute_tc.
constexpr int kFusedMaxBlocks = 512;
struct DispatchArgs {
  const char* x;              // [T, d] rows (read only when x_perm is set)
  int elt_bytes;
  int T, d, E, k, nblk, cap, renorm;
  const int32_t* idx;         // [T, k]
  const int32_t* lrank;       // [T, k]
  const int32_t* blk_counts;  // [E, nblk]
  int32_t* pos;               // [T, k]
  int32_t* src;               // [T * k]
  float* w;                   // [T, k], rewritten under a capacity
  char* x_perm;               // [T * k, d] or nullptr
  int32_t* offsets;           // [E + 1]
  int32_t* counts;            // [E]
  int32_t* user_counts;       // [E] or nullptr
  const float* blk_psum;      // [nblk, E]
  const float* blk_zsum;      // [nblk] or nullptr
  float *f, *p, *loss, *z_loss;
  int32_t* sk_flags;          // stream-K flags to clear, or nullptr
};
hipError_t launch_dispatch_tc(const DispatchArgs& a, hipStream_t s);

// Token choice: pos[t,j] = base + rank, src[pos] = t, x_perm[pos] = x[t]. With a
// capacity (cap < INT_MAX) slots ranked cap or later in their expert get pos = -1 and
// weight 0, and the token's kept weights w are renormalised when renorm is set.
// x_perm == nullptr: slots and weights only. sk_flags (or nullptr): the GEMMs' stream-K
// flags, cleared here.
hipError_t launch_permute_tc(const void* x, int elt_bytes, int T, int d, int E, int k,
                             const int32_t* idx, const int32_t* lrank, const int32_t* base,
                             const int32_t* offsets, int cap, int renorm, int32_t* pos,
                             int32_t* src, float* w, void* x_perm, int32_t* sk_flags,
                             hipStream_t s);

// Expert choice: row e*C + c takes token idx[e, c] (src; the row copy into x_perm only when
// x_perm is not nullptr). sk_flags as for launch_permute_tc.
hipError_t launch_permute_ec(const void* x, int elt_bytes, int d, int E, int C,
                             const int32_t* idx, int32_t* src, void* x_perm, int32_t* sk_flags,
                             hipStream_t s);

// Stream-K scratch of the bf16 grouped GEMMs (in the caller's workspace): partial sums, one
// slot of kStreamKSlotBytes per workgroup, and one int32 flag per workgroup, which must be
// zero when a GEMM starts (the permute kernels clear them; each GEMM leaves them zero).
// partial == nullptr: no stream-K (every tile whole).
constexpr int kStreamKSlots = 256;
constexpr size_t kStreamKSlotBytes = (size_t)256 * 256 * 4;  // a 256 x 256 fp32 tile
// Only tiles of at least this many K stages (of 32) are split: the down projection of a layer
// with d_ff < 32 * kStreamKMinStages never uses the scratch, which is then left out.
constexpr int kStreamKMinStages = 256;
struct StreamK {
  float* partial;   // [kStreamKSlots * kStreamKSlotBytes / 4]
  int32_t* flags;   // [kStreamKSlots]
};

// Grouped GEMMs over expert-contiguous rows (group e = rows [offsets[e], offsets[e+1])).
//   gate/up: h[r] = silu(A[r] W_gate[e]) * (A[r] W_up[e])  -> h [R, f]
//     A[r] = xp[gather[r]] (bf16 only: the rows are gathered from x inside the GEMM's loads;
//     every gather[r] * d must stay below 2^31) or xp[r] when gather is nullptr
//   down:    o[r] = h[r] W_down[e]                                   -> o [R, d] fp32
// With h_lo non-null (bf16 only) the gate/up epilogue also writes the bf16 rounding
// residual of h. With lo_rows > 0 (bf16 only) the down GEMM takes row r's residual from
// row r + lo_rows of h and writes o[r] = h[r] W_down[e] + h[r + lo_rows] W_down[e]
// (stream-K is then not used). R_max bounds the routed rows.
hipError_t launch_gemm_gateup(int bf16, const void* xp, const int32_t* gather, const void* Wgate,
                              const void* Wup, const int32_t* offsets, int E, int R_max, int d,
                              int f, void* h, void* h_lo, const StreamK& sk, hipStream_t s);
hipError_t launch_gemm_down(int bf16, const void* h, const void* Wdown, const int32_t* offsets,
                            int E, int R_max, int f, int d, float* o, int lo_rows,
                            const StreamK& sk, hipStream_t s);

// y[t] = sum_j w[t,j] * o[pos[t,j]]  (j in slot order)
hipError_t launch_combine_tc(const float* o, const int32_t* pos, const float* w, int T, int d,
                             int k, float* y, hipStream_t s);
// y[t] = sum over experts e (ascending) that chose t of score[e,c] * o[e*C + c]; else 0.
// runs: the select's run table (nullptr: each token searches the lists itself).
hipError_t launch_combine_ec(const float* o, const int32_t* idx, const float* score,
                             const int32_t* runs, int T, int d, int E, int C, float* y,
                             hipStream_t s);

// Per-block counts ([E, nblk]) and probability sums from router outputs (standalone aux loss).
hipError_t launch_aux_partials(const float* probs, const int32_t* idx, int T, int E, int k,
                               int32_t* blk_counts, float* blk_psum, hipStream_t s);
// f, p, loss (and optional counts) from per-block partials (E = 0: none of them), and
// z_loss = sum of blk_zsum / T when both are set.
hipError_t launch_aux_final(const int32_t* blk_counts, const float* blk_psum, int nblk, int T,
                            int E, int k, float* f, float* p, float* loss, int32_t* counts,
                            const float* blk_zsum, float* z_loss, hipStream_t s);
// Zero-fill helper (device memory), used for empty inputs.
hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t s);
