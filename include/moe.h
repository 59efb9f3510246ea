/*
 * moe.h — C ABI of the MI355X (gfx950) sparse Mixture-of-Experts layer forward.
 *
 * The layer (pages cited by title):
 *   - router: s = x W_g (+ b), g = softmax(s), TopK(g), y = sum_{i in TopK} g_i E_i(x)
 *     ("MoE" primer on qiita, section "ゲート / ルーターって何者？", the four router
 *     equations; bias as in "机器学习基础系列——混合专家模型", GatingNetwork);
 *     the selected weights renormalised to sum to 1 as in
 *     "Mixture of Experts（MoE）の理論と実装", MoELayer.route, and
 *     "Sparse Mixture of Experts(MoE) 아키텍처 심층 분석", TopKGating;
 *   - experts: E_i(x) = (silu(x W_gate) * (x W_up)) W_down, silu(z) = z / (1 + e^-z)
 *     ("Mixture of Experts（MoE）の理論と実装", Expert.forward; the Korean page's
 *     SwiGLUExpert);
 *   - load-balancing statistics f_i, p_i and loss = E * sum_i (f_i / k) p_i
 *     ("Mixture of Experts（MoE）の理論と実装", load_balancing_loss; the Korean page's
 *     compute_load_balancing_loss);
 *   - router z-loss z = mean_t (log sum_e exp(s_te))^2 over the router logits s (the
 *     Korean page's router_z_loss);
 *   - noisy top-k gating for training: s + softplus(x W_noise) * eps before the softmax
 *     (the Korean page's TopKGating, training branch), or s + eps (the fixed-scale noise
 *     of "机器学习基础系列——混合专家模型", MoELayer, with eps scaled by the caller);
 *   - expert-choice routing with capacity C = floor(T * cf / E): each expert takes the
 *     C tokens of largest softmax-over-tokens score (the Korean page's
 *     ExpertChoiceGating);
 *   - token choice with an expert capacity C = int((T / E) * cf * k): top-k routing as
 *     above, after which each expert keeps its first C assignments in token order and
 *     drops the rest; a token that lost a slot has its kept weights divided by their
 *     sum ("机器学习基础系列——混合专家模型", expert_capacity_routing).
 *
 * Conventions for every entry point:
 *   - All tensors are row-major and live in device memory (HBM) unless stated; the
 *     caller allocates every buffer, including the workspace. The library never
 *     allocates, frees, synchronises or keeps a pointer after it returns.
 *   - Work is enqueued on `stream` in order; results are valid once the caller
 *     synchronises that stream.
 *   - Activations and weights have the type `shape->dtype` (fp32 or bf16). Router
 *     logits, probabilities, gate weights, the output y and the statistics are fp32.
 *     bf16 products accumulate in fp32.
 *   - Every argument is checked on the host before any HIP call; a failed check
 *     returns a status and enqueues nothing. MOE_ERR_HIP reports a launch failure.
 *   - Token-choice slots list experts by descending probability, lower index first on
 *     ties. Expert-choice lists each expert's tokens in ascending token order; ties at
 *     the capacity boundary go to the lower token index.
 *   - Results are deterministic: the same inputs give bitwise the same outputs.
 *   - Entry points are reentrant; calls on different streams may overlap if their
 *     workspaces differ.
 *
 * Limits: 1 <= E <= 64; token choice 1 <= k <= min(E, 8); d_model and d_ff at most 2^20;
 * 0 <= T and T * max(k, 1) < 2^31; expert choice needs 1 <= C <= T and E * C < 2^31
 * (outside these: MOE_ERR_BAD_SHAPE). Limits of this implementation, not of the method,
 * return MOE_ERR_UNSUPPORTED: E > 64, k > 8, d_model or d_ff not a multiple of 64 (the
 * kernels run whole 64-column tiles), and fp32 layers with more than 64 * (65535 - E)
 * routed rows (T * k, or E * C). x, weights, y and the workspace must be 16-byte aligned.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_NULL_ARG = 1,            /* a required pointer is NULL */
  MOE_ERR_BAD_SHAPE = 2,           /* sizes out of range or inconsistent */
  MOE_ERR_UNSUPPORTED = 3,         /* valid request this library does not provide */
  MOE_ERR_WORKSPACE_TOO_SMALL = 4, /* ws_bytes < moe_workspace_size() */
  MOE_ERR_MISALIGNED = 5,          /* a pointer is not 16-byte aligned */
  MOE_ERR_HIP = 6                  /* a HIP launch failed */
} moe_status;

typedef enum moe_dtype { MOE_FP32 = 0, MOE_BF16 = 1 } moe_dtype;

/* MOE_TOKEN_CHOICE_CAPACITY is token choice (every "token choice" rule below applies)
 * with an expert capacity: see moe_capacity and moe_route. */
typedef enum moe_mode {
  MOE_TOKEN_CHOICE = 0,
  MOE_EXPERT_CHOICE = 1,
  MOE_TOKEN_CHOICE_CAPACITY = 2
} moe_mode;

/* Shape of one layer call. */
typedef struct moe_shape {
  int64_t T;             /* tokens (rows of x) */
  int64_t d_model;       /* width of x and y */
  int64_t d_ff;          /* hidden width of each expert */
  int32_t E;             /* experts */
  int32_t k;             /* token choice: experts per token; ignored in expert choice */
  int32_t mode;          /* moe_mode */
  int32_t dtype;         /* moe_dtype of x, W_g, W_gate, W_up, W_down */
  int32_t renormalize;   /* token choice: 1 = selected weights divided by their sum
                            (Mixture of Experts（MoE）の理論と実装, MoELayer.route);
                            0 = raw probabilities (the qiita router equations) */
  double capacity_factor; /* expert choice: C = floor(T * capacity_factor / E);
                             token choice with capacity: C = int((T / E) * capacity_factor
                             * k); both in double, > 0 and finite; ignored in plain token
                             choice */
} moe_shape;

/* Training noise of noisy top-k gating, token choice only (both token-choice modes).
 *   W_noise [d_model, E] dtype, layout of W_g; or NULL for additive noise
 *   eps     [T, E] fp32, the normal draw (one per token and expert); or NULL to have the
 *           router kernel draw it: eps[t, e] = scale * n(t, e) below
 *   seed, offset, scale   the in-kernel draw (ignored when eps is given); a non-finite
 *           scale returns MOE_ERR_BAD_SHAPE
 * The router's logits become s + softplus(x W_noise) * eps (softplus(z) = log(1 + e^z)),
 * or s + eps without W_noise, with s = x W_g (+ b_g): the Korean page's TopKGating
 * (training branch) and 机器学习基础系列——混合专家模型's MoELayer. Everything downstream —
 * softmax, top-k, weights, probs, counts, f, p, loss, z_loss — sees the noisy logits.
 * The in-kernel draw is counter-based, so that n(t, e) depends on (seed, offset, t, e)
 * only, not on the launch:
 *   (r0, r1, r2, r3) = Philox4x32-10 with counter (t, floor(e / 4), offset mod 2^32,
 *                      floor(offset / 2^32)) and key (seed mod 2^32, floor(seed / 2^32))
 *                      (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy
 *                      as 1, 2, 3", SC 2011)
 *   u_i = (floor(r_i / 2^8) + 1/2) / 2^24, strictly inside (0, 1)
 *   n(t, 4q + 2h + c) = sqrt(-2 ln u_{2h}) * (c = 0 ? cos : sin)(2 pi u_{2h+1})
 *                      (the Box-Muller transform, Box and Muller 1958)
 * evaluated in fp32 (the uniforms exactly; log, sqrt, cos and sin to about an ulp). A new
 * draw per training step takes a new offset (or seed). */
typedef struct moe_noise {
  const void* W_noise;
  const float* eps;
  uint64_t seed;
  uint64_t offset;
  float scale;
} moe_noise;

/* Human-readable name of a status code. Never NULL; the string is static. */
const char* moe_status_string(int32_t status);

/* Capacity C. Expert choice: floor(T * cf / E) (the Korean page's ExpertChoiceGating,
 * expert_capacity); MOE_ERR_BAD_SHAPE unless 1 <= C <= T. Token choice with capacity:
 * floor((T / E) * cf * k) evaluated in double in that order ("机器学习基础系列——混合专家
 * 模型", expert_capacity_routing); C = 0 is valid and drops every assignment. Host
 * only. Plain token choice returns MOE_ERR_BAD_SHAPE. */
moe_status moe_capacity(const moe_shape* shape, int64_t* capacity);

/* Bytes of device workspace moe_route / moe_forward / moe_aux_loss need for `shape`.
 * Host only; the same size serves all three entry points. */
moe_status moe_workspace_size(const moe_shape* shape, size_t* bytes);

/* Byte offset, inside the workspace, of an intermediate buffer of moe_forward, for
 * tests and debugging. After a moe_forward call has completed on the stream the
 * buffer holds that call's values until the workspace is used again. Host only.
 *   MOE_WS_OFFSETS [E+1] int32   first row of each expert's group; [E] = R
 *   MOE_WS_POS     [T, k] int32  token choice: row of each (token, slot), -1 when the
 *                                expert capacity dropped the slot
 *   MOE_WS_SRC     [R] int32     token of each row
 *   MOE_WS_XPERM   [R, d_model]  dtype, x rows in expert-contiguous order; only where rows are
 *                                copied: fp32, or T * d_model >= 2^31 (otherwise the gate/up
 *                                GEMM reads the rows of x through MOE_WS_SRC and this returns
 *                                MOE_ERR_UNSUPPORTED)
 *   MOE_WS_H       [R, d_ff]     dtype, silu(x W_gate) * (x W_up) per row
 *   MOE_WS_O       [R, d_model]  fp32, expert output per row (before weighting)
 * Expert choice in bf16 carries h's bf16 rounding residual: the MOE_WS_H region then holds
 * 2R rows (h, then the residual), and MOE_WS_O row r is the down projection of row r plus
 * that of row R + r.
 * R = T*k (token choice) or E*C (expert choice). With an expert capacity only rows
 * [0, offsets[E]) hold kept slots, offsets[E] = sum_e min(counts_e, C). MOE_WS_POS is
 * MOE_ERR_UNSUPPORTED in expert choice. */
enum {
  MOE_WS_OFFSETS = 0,
  MOE_WS_POS = 1,
  MOE_WS_SRC = 2,
  MOE_WS_XPERM = 3,
  MOE_WS_H = 4,
  MOE_WS_O = 5
};
moe_status moe_workspace_offset(const moe_shape* shape, int32_t which, size_t* offset);

/* Router (the qiita router equations; Mixture of Experts（MoE）の理論と実装,
 * MoELayer.route; the Korean page's TopKGating and ExpertChoiceGating).
 *   x      [T, d_model]   dtype
 *   W_g    [d_model, E]   dtype (the x @ W layout of MoELayer.__init__)
 *   b_g    [E] fp32 router bias added to the logits, or NULL for none
 *   noise  training noise (moe_noise), or NULL for none; MOE_ERR_UNSUPPORTED in expert
 *          choice
 * Token choice outputs:
 *   idx    [T, k] int32   selected experts, descending probability
 *   w      [T, k] fp32    gate weights of the selected experts
 * Expert choice outputs (C = moe_capacity):
 *   idx    [E, C] int32   tokens chosen by each expert, ascending token index
 *   w      [E, C] fp32    their scores (column-softmax values)
 * Optional outputs (NULL to skip):
 *   probs  [T, E] fp32    softmax probabilities (expert choice: over tokens, per column)
 *   counts [E] int32      assignments per expert (expert choice: C each)
 *   z_loss [1] fp32       router z-loss: mean over tokens of (log sum_e exp(s_te))^2, s the
 *                         logits with the bias (every mode; 0 when T = 0). Computed in the
 *                         router's pass over x: one fp32 log-partition per token, fixed-order
 *                         fp32 sums per 64 tokens, then an fp64 sum over those.
 * Token choice with capacity: idx and counts are those of plain token choice (counts
 * before any drop); w holds the weights after the capacity: 0 for a dropped slot, and
 * for a token that lost a slot its kept weights divided by their sum when renormalize
 * = 1 (a token that lost every slot gets zeros), unchanged when renormalize = 0. An
 * expert keeps the assignments of lowest token index; a token's slots go to distinct
 * experts, so the order of slots within a token decides nothing.
 * idx and w are required when T > 0 (with T = 0 there is nothing to write). */
moe_status moe_route(const moe_shape* shape, const void* x, const void* W_g, const float* b_g,
                     const moe_noise* noise, int32_t* idx, float* w, float* probs,
                     int32_t* counts, float* z_loss, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/* Whole layer forward ("Mixture of Experts（MoE）の理論と実装", MoELayer.forward: route,
 * run each expert on its tokens, add the weighted expert outputs; the Korean page's
 * MoELayerWithAuxLoss, which also returns the load-balancing loss): router, dispatch
 * (histogram, prefix sum, stable permutation of token rows into expert-contiguous order),
 * grouped SwiGLU gate/up GEMM, grouped down GEMM, weighted combine, and (token choice) the
 * load-balancing statistics.
 *   x, W_g, b_g, noise   as in moe_route
 *   W_gate, W_up  [E, d_model, d_ff] dtype, expert e's matrix at offset e*d_model*d_ff
 *   W_down        [E, d_ff, d_model] dtype
 *   y             [T, d_model] fp32   y_t = sum over the token's experts of
 *                 weight * E_e(x_t); in expert choice a token no expert takes gets 0
 * Optional outputs (NULL to skip): idx, w, probs, counts, z_loss as in moe_route, and,
 * token choice only (with capacity: computed from the assignments before any drop):
 *   f     [E] fp32   counts / T (sums to k)
 *   p     [E] fp32   mean over tokens of probs
 *   loss  [1] fp32   E * sum_e (f_e / k) * p_e (1 under uniform routing)
 * Passing f, p or loss in expert-choice mode returns MOE_ERR_UNSUPPORTED: the pages
 * define these statistics for token choice only.
 * Precision (bf16): the hidden activation h = silu(x W_gate) * (x W_up) is formed in fp32
 * and rounded to bf16 for the down projection. In expert choice the bf16 rounding
 * residual of h is carried as a second bf16 term (h ~ h_hi + h_lo): expert-choice scores
 * span a wide range across tokens, and a single rounding of h would cost about 2.5% of
 * the output RMS on the 16-expert workload; the pair doubles the down projection's
 * multiply work (each tile takes 128 tokens' rows and their residual rows, and sums the
 * two products before storing o). */
moe_status moe_forward(const moe_shape* shape, const void* x, const void* W_g, const float* b_g,
                       const moe_noise* noise, const void* W_gate, const void* W_up,
                       const void* W_down, float* y,
                       int32_t* idx, float* w, float* probs, int32_t* counts, float* f, float* p,
                       float* loss, float* z_loss, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): moe_forward with the same arguments
 * and results, minus the workspace. The workspace is a file-scope device array of
 * MOE_NOALLOC_SCRATCH_BYTES (256 MiB) inside the library, one per GPU, held until the
 * process ends; its address is looked up (hipGetSymbolAddress) on the first call on each
 * device. The call allocates nothing (no hipMalloc, no library allocation).
 *   - Shapes whose moe_workspace_size exceeds MOE_NOALLOC_SCRATCH_BYTES return
 *     MOE_ERR_WORKSPACE_TOO_SMALL before any HIP call (every other check is moe_forward's).
 *   - Every call on one GPU shares that GPU's array, which keeps the last call's
 *     intermediates: calls that overlap on one GPU (different streams, or threads) race and
 *     must be ordered by the caller. Nothing in the array needs to start at zero.
 *   - MOE_ERR_HIP also reports a failed lookup of the array's address. */
#define MOE_NOALLOC_SCRATCH_BYTES (256u << 20)
moe_status moe_forward_noalloc(const moe_shape* shape, const void* x, const void* W_g,
                               const float* b_g, const moe_noise* noise, const void* W_gate,
                               const void* W_up, const void* W_down, float* y, int32_t* idx,
                               float* w, float* probs, int32_t* counts, float* f, float* p,
                               float* loss, float* z_loss, hipStream_t stream);

/* Load-balancing statistics from router outputs (Mixture of Experts（MoE）の理論と実装,
 * load_balancing_loss; the Korean page's compute_load_balancing_loss), token choice:
 *   probs [T, E] fp32, idx [T, k] int32 (values in [0, E)) ->
 *   f [E] = counts / T, p [E] = mean_t probs, loss [1] = E * sum (f / k) p,
 *   counts [E] int32 (optional, NULL to skip).
 * Expert-choice shapes return MOE_ERR_UNSUPPORTED. With T = 0, f, p, loss and counts
 * are zero. */
moe_status moe_aux_loss(const moe_shape* shape, const float* probs, const int32_t* idx, float* f,
                        float* p, float* loss, int32_t* counts, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* Stage timing. While enabled, every moe_route / moe_forward / moe_aux_loss call
 * records a hipEvent pair around each stage's kernel launch on the caller's stream.
 * moe_profile_read waits for the recorded events, returns per-stage totals
 * (milliseconds, and the number of timed launches) for stages 0..n-1 and clears them.
 * Not thread-safe: one profiling caller per process. */
enum {
  MOE_STAGE_ROUTER = 0,
  MOE_STAGE_SCAN = 1,
  MOE_STAGE_PERMUTE = 2,
  MOE_STAGE_GEMM_GATE_UP = 3,
  MOE_STAGE_GEMM_DOWN = 4,
  MOE_STAGE_COMBINE = 5,
  MOE_STAGE_AUX = 6,
  MOE_STAGE_EC_SELECT = 7,
  MOE_NUM_STAGES = 8
};
moe_status moe_profile_enable(int32_t on);
moe_status moe_profile_read(double* total_ms, int64_t* launches, int32_t n);
const char* moe_stage_name(int32_t stage);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
