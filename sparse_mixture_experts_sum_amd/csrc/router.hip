// Router kernels for gfx950.
//
// Token choice (qiita primer, router equations s = W_g x, g = softmax(s), TopK(g);
// "Mixture of Experts（MoE）の理論と実装", MoELayer.route; the Korean page's
// TopKGating): one workgroup takes 64 tokens. The skinny GEMM x W_g runs on
// 16x16 MFMA tiles (x rows streamed from HBM straight into registers as the A
// operand, W_g staged in LDS as the B operand: bf16 copied as it lies and read with
// transposing LDS reads, otherwise transposed through registers), then four threads per
// token do the max-shifted softmax, top-k by (logit desc, index asc) and the
// weights. The same workgroup counts its slots per expert, ranks each slot among
// the block's slots of the same expert (flattened token-major order) and sums the
// block's probabilities per expert, so dispatch and the aux statistics need no
// second pass over the routing.
//
// Expert choice (the Korean page's ExpertChoiceGating): the same GEMM writes the
// logits transposed, [E, T]; a second kernel takes one expert per workgroup.
//
// Noisy top-k gating (the Korean page's TopKGating, training branch): the noise
// projection x W_noise runs as E more MFMA columns over the same x fragments (W_noise
// staged beside W_g), and each logit becomes s + softplus(x W_noise) * eps before the
// softmax. eps, the normal draw, is an input, or is drawn here, per (token, expert), from a
// counter-based generator (Philox4x32-10 and the Box-Muller transform), so that no draw
// travels through HBM. Without W_noise the draw is added as is (the fixed-scale noise of
// 机器学习基础系列——混合专家模型, MoELayer).
#include <float.h>
#include <limits.h>

#include "common.h"
#include "kernels.h"

namespace {

template <typename TI>
struct RouterMma;

template <>
struct RouterMma<bf16> {
  static constexpr int VEC = 8;  // elements per 16-byte chunk
  __device__ static void step(f32x4& acc, u32x4 a, u32x4 b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
};

template <>
struct RouterMma<float> {
  static constexpr int VEC = 4;
  __device__ static void step(f32x4& acc, u32x4 a, u32x4 b) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[q]), __uint_as_float(b[q]),
                                                 acc, 0, 0, 0);
  }
};

constexpr int kRT = kRouterTokens;  // tokens per workgroup (4 waves x 16)

// Workgroup barrier after this wave's LDS accesses have completed; unlike __syncthreads
// it does not wait for outstanding global loads.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}
constexpr int kRouterWgBytes = 131072;  // LDS for the transposed W_g slice
constexpr int kRouterPF = 4;            // iterations of x loads in flight per wave

// x chunks of iteration `it` of a stage: lane group g takes chunks 4u + g, u = 0..3 (the
// k ranges of the four 32-deep MFMA steps). Loads stay in bounds (clamped to the last
// chunk of the stage, in the same row) and are always issued, so that the compiler sees
// the same number of loads in flight on every path; the loop then runs whole groups of
// PF iterations with no branch. The data is used as loaded: chunks past the stage's end
// meet a zero W_g fragment in the MFMA instead (see the loop). Masking the loaded
// values here would make the compiler wait for every load in flight, prefetches
// included, at each group's end.
template <int VEC, typename TI>
__device__ __forceinline__ void router_load_x(const TI* xs, int it, int kn, int g,
                                              u32x4 (&av)[4]) {
  constexpr int ITK = 16 * VEC;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int kx = it * ITK + (4 * u + g) * VEC;
    av[u] = ld16(xs + min(kx, kn - VEC));
  }
}

// Stage W_g[kc : kc + kn, 0 : E) transposed into LDS (row n = expert, LDW elements per
// row). bf16 with E a multiple of 8: each thread reads 8 k-rows x 8 experts (8 x 16
// bytes), transposes the block in registers (v_perm_b32 picks the low or high halves of
// two dwords) and writes 8 rows of 16 bytes; otherwise element by element.
template <typename TI>
__device__ __forceinline__ void stage_wg_transposed(const TI* __restrict__ src, int kn, int E,
                                                    int LDW, TI* Wl, int tid) {
  if constexpr (sizeof(TI) == 2) {
    if (E % 8 == 0 && kn % 8 == 0) {
      const int eb8 = E / 8, nblk = (kn / 8) * eb8;
      for (int bi = tid; bi < nblk; bi += 256) {
        const int k0 = (bi / eb8) * 8, e0 = (bi % eb8) * 8;
        u32x4 c[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = ld16(src + (size_t)(k0 + i) * E + e0);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          u32x4 o;
#pragma unroll
          for (int j = 0; j < 4; ++j) o[j] = __builtin_amdgcn_perm(c[2 * j + 1][e >> 1], c[2 * j][e >> 1], sel);
          st16(Wl + (size_t)(e0 + e) * LDW + k0, o);
        }
      }
      return;
    }
  }
  constexpr int VEC = 16 / (int)sizeof(TI);
  const int nchunk = kn * E / VEC;
  for (int c = tid; c < nchunk; c += 256) {
    u32x4 v = ld16(src + (size_t)c * VEC);
    const TI* ve = reinterpret_cast<const TI*>(&v);
#pragma unroll
    for (int q = 0; q < VEC; ++q) {
      const int flat = c * VEC + q;
      const int kk = flat / E, n = flat - kk * E;
      Wl[n * LDW + kk] = ve[q];
    }
  }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// s_waitcnt with only vmcnt constrained (expcnt and lgkmcnt left at their maximum)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// bf16 with E a multiple of 8: W_g[kc : kc + kn, 0 : E) copied as it lies in HBM (kn rows
// of E elements, 2E bytes each) into LDS at dst by direct global->LDS loads, 1 KB per wave
// instruction, lane l's 16 bytes into slot l (kn * E * 2 is a whole number of KB: kn is a
// multiple of 64). No registers in between: the B fragments come out of LDS with
// transposing reads (wg_fragment).
__device__ __forceinline__ void stage_wg_direct(const bf16* __restrict__ src, int kn, int E,
                                                char* dst, int wave, int lane) {
  const int nchunk = kn * E / 8;  // 16-byte chunks
  const int ninst = (nchunk + 63) / 64;
  for (int j = wave; j < ninst; j += 4) {
    const int c = min(64 * j + lane, nchunk - 1);
    __builtin_amdgcn_global_load_lds(src + (size_t)c * 8, (lds_void*)(dst + j * 1024), 16, 0, 0);
  }
}

// B fragment of a 16x16x32 MFMA from the natural layout of stage_wg_direct: 8 consecutive
// k (rows kr .. kr + 7) of column col0 + lane % 16, from two transposing reads. Source lane
// i of each 16-lane group addresses row kr + i / 4 (+ 4 for the second read), columns
// col0 + 4 (i % 4) .. + 3; result lane j gets column col0 + j of the four rows. Columns at
// or past E read the next row's values (the logits of padding experts are never used).
__device__ __forceinline__ u32x4 wg_fragment(const char* w, int rowbytes, int kr, int col0,
                                             int lane) {
  const int i = lane & 15;
  const char* p = w + (size_t)(kr + (i >> 2)) * rowbytes + (col0 + 4 * (i & 3)) * 2;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * rowbytes));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(u32x4, v);
}

// softplus(z) = log(1 + e^z), as max(z, 0) + log(1 + e^-|z|) so that e^z never overflows
__device__ __forceinline__ float softplus_f(float z) {
  return fmaxf(z, 0.f) + log1pf(expf(-fabsf(z)));
}

// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2,
// 3", SC 2011): ten rounds of two 32 x 32 -> 64-bit products on the counter, with a Weyl
// sequence on the key between rounds.
__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    if (i) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0], p1 = (uint64_t)0xCD9E8D57u * c[2];
    c = u32x4{(uint32_t)(p1 >> 32) ^ c[1] ^ k0, (uint32_t)p1, (uint32_t)(p0 >> 32) ^ c[3] ^ k1,
              (uint32_t)p0};
  }
  return c;
}

// The in-kernel normal draw n(t, e): Philox4x32-10 of counter (t, e / 4, offset) under key
// seed gives four words r_0..r_3; u_i = (j_i + 1/2) / 2^24 with j_i = r_i / 256 (integer
// part), strictly inside (0, 1); the Box-Muller transform (Box and Muller, 1958) of the pair
// (u_0, u_1), sqrt(-2 ln u_0) times cos or sin of 2 pi u_1, gives experts 4q and 4q + 1
// (cosine, sine), of (u_2, u_3) experts 4q + 2 and 4q + 3.
// u_i takes 25 significant bits once j_i >= 2^23, so it is not an fp32 value there; its
// complement 1 - u_i = (2^24 - j_i - 1/2) / 2^24 is, and so ln u_0 = log1p(-(1 - u_0)) is
// evaluated from it, and the angle through cos(pi (2 - a)) = cos(pi a), sin(pi (2 - a)) =
// -sin(pi a) with 2 - a = 2 (1 - u_1) half turns. Every argument is then exact, and the
// draw differs from its definition only by the fp32 math functions' own rounding.
__device__ __forceinline__ float noise_draw(const RouterArgs& a, int t, int e) {
  const u32x4 r = philox4x32_10(u32x4{(uint32_t)t, (uint32_t)(e >> 2), a.off_lo, a.off_hi},
                                a.seed_lo, a.seed_hi);
  const int h = (e >> 1) & 1;
  const uint32_t j0 = (h ? r[2] : r[0]) >> 8, j1 = (h ? r[3] : r[1]) >> 8;
  constexpr uint32_t kHalf = 1u << 23;
  // exact: (j + 1/2) below 2^23, (2^24 - j - 1/2) from 2^23 on, both at most 24 bits
  const float lnu0 = j0 < kHalf ? logf(((float)j0 + 0.5f) * 0x1p-24f)
                                : log1pf(-(((float)((1u << 24) - j0) - 0.5f) * 0x1p-24f));
  const bool up = j1 >= kHalf;
  const float turns = up ? ((float)((1u << 24) - j1) - 0.5f) * 0x1p-23f  // 2 - 2 u_1
                         : ((float)j1 + 0.5f) * 0x1p-23f;                // 2 u_1
  const float rad = sqrtf(-2.0f * lnu0);
  if (e & 1) {
    const float sv = sinpif(turns);
    return rad * (up ? -sv : sv);
  }
  return rad * cospif(turns);
}

// NOISE: 0 none, 1 eps added to the logits, 2 softplus(x W_noise) * eps added; eps from
// a.eps, or drawn (noise_draw, times a.noise_scale) when a.eps is null.
// DIRECT (bf16, E a multiple of 8): W_g (and W_noise) staged by stage_wg_direct and read
// with wg_fragment; otherwise transposed through registers by stage_wg_transposed.
template <typename TI, int EP, int NOISE, bool DIRECT>
__global__ __launch_bounds__(256) void router_kernel(RouterArgs a, int ec) {
  using M = RouterMma<TI>;
  constexpr int VEC = M::VEC;
  constexpr int ITK = 16 * VEC;                                  // k per iteration
  constexpr int NG = EP / 16;                                    // 16-column blocks of W_g
  constexpr int NB = NOISE == 2 ? 2 * NG : NG;                   // plus those of W_noise
  constexpr int KC = kRouterWgBytes / (NB * 16 * (int)sizeof(TI));  // k per LDS stage
  constexpr int LDW = KC + 16 / (int)sizeof(TI);                 // padded row (16 bytes)
  constexpr int LSP = EP + 1;
  constexpr int PF = kRouterPF;
  static_assert(KC % ITK == 0, "stage must hold whole iterations");
  static_assert(!DIRECT || sizeof(TI) == 2, "direct staging is the bf16 layout");
  // DIRECT: W_noise sits after W_g's KC rows of EP elements (the same split as the
  // transposed layout's)
  constexpr int WN_BYTES = KC * EP * 2;

  // rows [0, EP): W_g transposed; rows [EP, 2 EP): W_noise transposed (NOISE == 2).
  // DIRECT: W_g's [k, E] rows from byte 0, W_noise's from byte WN_BYTES.
  __shared__ __attribute__((aligned(16))) TI Wl[NB * 16 * LDW];
  __shared__ float Ls[kRT * LSP];
  __shared__ float red[256];
  __shared__ float zred[4];
  __shared__ float bias_s[64];
  __shared__ int sel[kRT * 8];
  __shared__ int running[64];

  const TI* __restrict__ x = static_cast<const TI*>(a.x);
  const TI* __restrict__ Wg = static_cast<const TI*>(a.Wg);
  const int T = a.T, d = a.d, E = a.E;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4;
  const int t0 = blockIdx.x * kRT;
  const int trow = t0 + wave * 16 + (lane & 15);
  const TI* xrow = x + (size_t)min(trow, T - 1) * d;

  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the bias is loaded now and stored to LDS after the logits pass, so that its load
  // latency hides behind that pass
  const float bias_r = (a.bias && tid < E) ? a.bias[tid] : 0.f;
  // so is the noise draw of this lane's logits: token wave*16 + 4g + r, expert
  // nb*16 + lane%16 (the accumulator layout below)
  float epsv[NOISE ? NG : 1][4];
  if constexpr (NOISE != 0) {
#pragma unroll
    for (int nb = 0; nb < NG; ++nb) {
      const int e = nb * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + wave * 16 + 4 * g + r;
        epsv[nb][r] = (t < T && e < E)
                          ? (a.eps ? a.eps[(size_t)t * E + e] : a.noise_scale * noise_draw(a, t, e))
                          : 0.f;
      }
    }
  }

  // W_g is staged transposed in LDS (one slice of up to KC rows of k at a time; at most
  // a few slices: d / KC); x is streamed from HBM into registers, PF iterations ahead.
  // B fragments of padding experts (>= E) read expert E-1's row (their logits are never
  // used); x and W_g reads past the slice's last k are clamped into it, and the W_g
  // fragment of such a k is replaced by zeros.
  for (int kc = 0; kc < d; kc += KC) {
    const int kn = min(KC, d - kc);
    // the first x loads of the slice go out before W_g is staged, so that the two
    // latencies overlap (the barriers below wait for LDS work only, not for loads)
    const TI* xs = xrow + kc;
    const int nit = (kn + ITK - 1) / ITK;
    u32x4 av[PF][4];
    if constexpr (DIRECT) {
      // the slice's direct loads go out first, then the first x loads: waiting for the
      // former (loads complete in order) does not wait for the latter
      if (kc > 0) lds_barrier();  // the previous slice's fragment reads are done
      // (a uniform wave index keeps the loads' LDS destinations scalar)
      const int wave_u = __builtin_amdgcn_readfirstlane(wave);
      stage_wg_direct(reinterpret_cast<const bf16*>(Wg) + (size_t)kc * E, kn, E,
                      reinterpret_cast<char*>(Wl), wave_u, lane);
      if constexpr (NOISE == 2)
        stage_wg_direct(static_cast<const bf16*>(a.Wn) + (size_t)kc * E, kn, E,
                        reinterpret_cast<char*>(Wl) + WN_BYTES, wave_u, lane);
#pragma unroll
      for (int p = 0; p < PF - 1; ++p) router_load_x<VEC>(xs, p, kn, g, av[p]);
      // this wave's share of the slice has landed (the x loads behind it may still be in
      // flight); then every wave's has. A plain barrier: a fence would wait for the x
      // loads too.
      wait_vmcnt<(PF - 1) * 4>();
      __builtin_amdgcn_s_barrier();
    } else {
#pragma unroll
      for (int p = 0; p < PF - 1; ++p) router_load_x<VEC>(xs, p, kn, g, av[p]);
      lds_barrier();  // the previous slice's fragment reads are done
      stage_wg_transposed<TI>(Wg + (size_t)kc * E, kn, E, LDW, Wl, tid);
      if constexpr (NOISE == 2)
        stage_wg_transposed<TI>(static_cast<const TI*>(a.Wn) + (size_t)kc * E, kn, E, LDW,
                                Wl + EP * LDW, tid);
      lds_barrier();  // the slice is in LDS
    }
    for (int it0 = 0; it0 < nit; it0 += PF) {
#pragma unroll
      for (int j = 0; j < PF; ++j) {
        const int it = it0 + j;
        router_load_x<VEC>(xs, it + PF - 1, kn, g, av[(j + PF - 1) % PF]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int kx = it * ITK + (4 * u + g) * VEC;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            u32x4 bw;
            if constexpr (DIRECT) {
              // W_noise blocks (nb >= NG) sit WN_BYTES further on
              bw = wg_fragment(reinterpret_cast<const char*>(Wl) + (nb >= NG ? WN_BYTES : 0),
                               2 * E, min(kx, kn - VEC), (nb % NG) * 16, lane);
            } else {
              // W_noise blocks (nb >= NG) sit EP rows further down
              const int row = (nb >= NG ? EP : 0) + min((nb % NG) * 16 + (lane & 15), E - 1);
              bw = ld16(&Wl[row * LDW + min(kx, kn - VEC)]);
            }
            const u32x4 bv = kx < kn ? bw : u32x4{0u, 0u, 0u, 0u};  // k past the stage: 0
            M::step(acc[nb], av[j][u], bv);
          }
        }
      }
    }
  }

  if (tid < 64) bias_s[tid] = bias_r;
  __syncthreads();
  // acc[nb][r] = logit of token (wave*16 + 4g + r), expert (nb*16 + lane%16)
  if (ec) {
#pragma unroll
    for (int nb = 0; nb < EP / 16; ++nb) {
      const int e = nb * 16 + (lane & 15);
      if (e >= E) continue;
      const float bz = bias_s[e];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + wave * 16 + 4 * g + r;
        if (t < T) a.logitsT[(size_t)e * T + t] = acc[nb][r] + bz;
      }
    }
    if (!a.blk_zsum) return;  // else on to the per-token log-partition below
  }

  // logits with the bias (and the training noise) into LDS; padding experts (>= E) have
  // bias 0 and are never read
#pragma unroll
  for (int nb = 0; nb < NG; ++nb) {
    const float bz = bias_s[nb * 16 + (lane & 15)];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = acc[nb][r] + bz;
      if constexpr (NOISE == 1) v += epsv[nb][r];
      if constexpr (NOISE == 2) v += softplus_f(acc[NG + nb][r]) * epsv[nb][r];
      Ls[(wave * 16 + 4 * g + r) * LSP + nb * 16 + (lane & 15)] = v;
    }
  }
  if (tid < 64) running[tid] = 0;
  __syncthreads();

  // ---- softmax and top-k: four threads per token, thread `part` owns experts part+4i
  constexpr int PER = EP / 4;
  const int tok = tid >> 2, part = tid & 3;
  const int t = t0 + tok;
  const bool valid = t < T;
  const int k = a.k;
  float lv[PER];
  float lmax = -FLT_MAX;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = part + 4 * i;
    lv[i] = -FLT_MAX;
    if (e < E) {
      lv[i] = Ls[tok * LSP + e];
      lmax = fmaxf(lmax, lv[i]);
    }
  }
  lmax = fmaxf(lmax, __shfl_xor(lmax, 1));
  lmax = fmaxf(lmax, __shfl_xor(lmax, 2));
  float ex[PER];
  float lsum = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = part + 4 * i;
    ex[i] = e < E ? expf(lv[i] - lmax) : 0.f;
    lsum += ex[i];
  }
  lsum += __shfl_xor(lsum, 1);
  lsum += __shfl_xor(lsum, 2);

  // z-loss partial: sum over the block's tokens of (log sum_e exp(s_e))^2, in a fixed
  // order (xor tree over the 16 tokens of a wave, then the four waves in order)
  if (a.blk_zsum) {
    const float lse = lmax + logf(lsum);
    float zv = (valid && part == 0) ? lse * lse : 0.f;
#pragma unroll
    for (int off = 4; off < 64; off <<= 1) zv += __shfl_xor(zv, off);
    if (lane == 0) zred[wave] = zv;
    if (ec) {
      __syncthreads();
      if (tid == 0) a.blk_zsum[blockIdx.x] = ((zred[0] + zred[1]) + zred[2]) + zred[3];
      return;
    }
  }

  // top-k by (logit desc, expert asc); every thread of the token ends with the same picks
  uint32_t taken = 0;
  float selp[8];
  int sele[8];
  for (int j = 0; j < k; ++j) {
    float bv = -FLT_MAX;
    int be = INT_MAX;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = part + 4 * i;
      if (e < E && !((taken >> i) & 1u) && (be == INT_MAX || lv[i] > bv)) {
        bv = lv[i];
        be = e;
      }
    }
#pragma unroll
    for (int o = 1; o <= 2; o <<= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oe = __shfl_xor(be, o);
      if (oe != INT_MAX && (be == INT_MAX || ov > bv || (ov == bv && oe < be))) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 3) == part) taken |= 1u << (be >> 2);
    sele[j] = be;
    selp[j] = expf(bv - lmax) / lsum;
  }
  if (valid) {
    float den = 0.f;
    if (a.renorm)
      for (int j = 0; j < k; ++j) den += selp[j];
    for (int j = part; j < k; j += 4) {
      a.idx[(size_t)t * k + j] = sele[j];
      a.w[(size_t)t * k + j] = a.renorm ? selp[j] / den : selp[j];
    }
    if (part == 0)
      for (int j = 0; j < k; ++j) sel[tok * k + j] = sele[j];
  }
  // probabilities: to HBM (optional) and into the block's per-expert sums
  float pv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = part + 4 * i;
    pv[i] = 0.f;
    if (e < E) {
      const float pe = ex[i] / lsum;
      if (valid && a.probs) a.probs[(size_t)t * E + e] = pe;
      pv[i] = valid ? pe : 0.f;
    }
  }
  block_expert_sums<PER>(pv, PER, E, red, a.blk_psum + (size_t)blockIdx.x * E);
  // (block_expert_sums' barrier also orders the zred writes above before this read)
  if (a.blk_zsum && tid == 0) a.blk_zsum[blockIdx.x] = ((zred[0] + zred[1]) + zred[2]) + zred[3];

  const int nvalid = min(kRT, T - t0);
  // slot ranks within the block: wave 0 walks the slots in flattened order, 64 at a time
  if (wave == 0) {
    const int nent = nvalid * k;
    const uint64_t below = (1ull << lane) - 1ull;
    for (int c0 = 0; c0 < nent; c0 += 64) {
      const int q = c0 + lane;
      const bool act = q < nent;
      const int e = act ? sel[q] : 0;
      uint64_t m = __ballot(act);
#pragma unroll
      for (int b = 0; b < 6; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t bb = __ballot(act && bit);
        m &= bit ? bb : ~bb;
      }
      const int before = __popcll(m & below);
      const int r = act ? running[e] + before : 0;
      __builtin_amdgcn_wave_barrier();
      if (act && before == 0) running[e] += __popcll(m);
      if (act) a.lrank[(size_t)t0 * k + q] = r;
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();
  if (tid < E) a.blk_counts[(size_t)tid * gridDim.x + blockIdx.x] = running[tid];
}

// ---------------------------------------------------------------------------------
// Expert choice: one workgroup (1024 threads) per expert.
//   column max, min and sum of exp over the expert's T logits (fixed-order reductions),
//   the C-th largest logit key: one histogram pass over value buckets (monotone in the
//   logit) and a direct rank of the chosen bucket's keys, or, for a wide bucket, a radix
//   select (4 x 8 bits of the key, most significant first); then a stable compaction in
//   token order: every key above the threshold plus the first (C - above) keys equal to
//   it.
// Each thread owns a contiguous run of ceil(T / 1024) tokens and reads their logits from
// HBM once, into registers (PER > 0 of them: T <= 1024 PER), which every pass after that
// reuses. Up to 32768 tokens (PER < 0) the column is staged in LDS instead, thread-major
// (a thread's j-th token at j * 1024 + thread), so that a pass's reads are consecutive
// across lanes; longer columns read HBM in every pass (PER = 0). (Staged token-major, the
// reads of a thread's consecutive tokens hit the same LDS banks many times over: 1.3-2.6 us
// per pass at 8192 tokens.) Each wave counts into its own histogram (the logits of one
// expert share their leading key bits, so one shared histogram would take thousands of
// same-address atomics), and wave 0 finds the bucket holding the C-th key with a prefix
// sum across its lanes.
// ---------------------------------------------------------------------------------
constexpr int kEcThreads = 1024;
constexpr int kEcWaves = kEcThreads / 64;
constexpr int kEcCand = kEcThreads;  // keys of the selected value bucket ranked directly
constexpr int kEcLdsTokens = 32768;

template <int PER>
__global__ __launch_bounds__(kEcThreads) void ec_select_kernel(const float* __restrict__ logitsT,
                                                               int T, int E, int C, int32_t* idx,
                                                               float* score, float* probs,
                                                               int32_t* offsets, int32_t* counts,
                                                               int32_t* src,
                                                               int32_t* sk_flags,
                                                               int32_t* runs) {
  constexpr bool INLDS = PER < 0;
  __shared__ float colsh[INLDS ? kEcLdsTokens : 1];
  __shared__ int whist[kEcWaves][256];
  __shared__ float redf[kEcWaves];
  __shared__ long long scan_sh[17];
  __shared__ float redlo[kEcWaves];
  __shared__ float redsum[kEcWaves];
  __shared__ int sel_digit, sel_need, sel_cnt;
  __shared__ uint32_t cand_key[kEcCand];
  __shared__ int cand_above[kEcCand];
  __shared__ int cand_n, cand_sel;
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const float* col = logitsT + (size_t)e * T;
  if (sk_flags && e == 0)
    for (int i = tid; i < kStreamKSlots; i += kEcThreads) sk_flags[i] = 0;

  // contiguous token range of this thread
  const int per = (T + kEcThreads - 1) / kEcThreads;
  const int tb = min(T, tid * per), te = min(T, tb + per);
  const int nt = te - tb;
  float lv[PER > 0 ? PER : 1];
  if constexpr (PER > 0) {
    if (nt == PER && (reinterpret_cast<uintptr_t>(col + tb) & 15) == 0) {
#pragma unroll
      for (int j = 0; j < PER; j += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(col + tb + j);
#pragma unroll
        for (int i = 0; i < 4; ++i) lv[j + i] = v[i];
      }
    } else {
#pragma unroll
      for (int j = 0; j < PER; ++j) lv[j] = j < nt ? col[tb + j] : 0.f;
    }
  }
  if constexpr (INLDS) {
    for (int t = tid; t < T; t += kEcThreads) {
      const int owner = t / per;
      colsh[(t - owner * per) * kEcThreads + owner] = col[t];
    }
    __syncthreads();
  }
  // f(t, logit) over this thread's tokens, in token order
  auto each = [&](auto&& f) {
    if constexpr (PER > 0) {
#pragma unroll
      for (int j = 0; j < PER; ++j)
        if (j < nt) f(tb + j, lv[j]);
    } else if constexpr (INLDS) {
      for (int j = 0; j < nt; ++j) f(tb + j, colsh[j * kEcThreads + tid]);
    } else {
      for (int t = tb; t < te; ++t) f(t, col[t]);
    }
  };

  // column max, min and softmax sum in one pass and one barrier: each thread sums
  // exp(l - its own max), each wave rescales its lanes' sums to the wave max, and the
  // wave sums are rescaled to the column max in wave order (a fixed order)
  float m = -FLT_MAX, lo = FLT_MAX;
  each([&](int, float l) {
    m = fmaxf(m, l);
    lo = fminf(lo, l);
  });
  float s = 0.f;
  each([&](int, float l) { s += expf(l - m); });
  {
    const float mw = warp_max(m);
    s *= expf(m - mw);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) s += __shfl_xor(s, o);
    m = mw;
  }
  lo = -warp_max(-lo);
  if (lane == 0) {
    redf[wid] = m;
    redlo[wid] = lo;
    redsum[wid] = s;
  }
  __syncthreads();
  m = redf[0];
  lo = redlo[0];
  for (int i = 1; i < kEcWaves; ++i) {
    m = fmaxf(m, redf[i]);
    lo = fminf(lo, redlo[i]);
  }
  float sum = 0.f;
  for (int i = 0; i < kEcWaves; ++i) sum += redsum[i] * expf(redf[i] - m);

  // The C-th largest key (float_key order), `thr`, and how many keys equal to it are taken,
  // `need`. Histograms count keys per bucket in per-wave LDS arrays; wave 0 then walks the
  // 256 buckets from the top (lane l owns buckets 255 - 4l .. 252 - 4l) to the one holding
  // the need-th largest remaining key.
  auto find_bucket = [&](int need_in) {
    if (wid == 0) {
      int c[4], cl = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int dg = 255 - 4 * lane - j;
        int v = 0;
        for (int w = 0; w < kEcWaves; ++w) v += whist[w][dg];
        c[j] = v;
        cl += v;
      }
      int incl = cl;  // keys in buckets above and at this lane's (inclusive scan)
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o);
        if (lane >= o) incl += u;
      }
      const int excl = incl - cl;
      if (excl < need_in && need_in <= incl) {  // exactly one lane: the key is here
        int cum = excl, j = 0;
        for (; j < 3; ++j) {
          if (cum + c[j] >= need_in) break;
          cum += c[j];
        }
        sel_digit = 255 - 4 * lane - j;
        sel_need = need_in - cum;
        sel_cnt = c[j];
      }
    }
    __syncthreads();
  };
  uint32_t prefix = 0;
  int need = C;
  bool found = false;
  // Value buckets: bucket(l) = floor((l - min) * 256 / (max - min)), clamped, is monotone in
  // l, so the key sits in the bucket where the count from the top reaches C. Its keys (at
  // most kEcCand) are then ranked among themselves, one per thread. Columns whose span is
  // not a finite positive number, or whose bucket holds more keys (many equal logits), take
  // the radix passes below.
  const float span = m - lo;
  const float scale = 256.0f / span;
  if (isfinite(span) && span > 0.f && isfinite(scale)) {
    auto bucket = [&](float l) { return (int)fminf(fmaxf((l - lo) * scale, 0.f), 255.f); };
    for (int i = lane; i < 256; i += 64) whist[wid][i] = 0;
    __builtin_amdgcn_wave_barrier();
    each([&](int, float l) { atomicAdd(&whist[wid][bucket(l)], 1); });
    __syncthreads();
    find_bucket(need);
    const int sb = sel_digit, sneed = sel_need, scnt = sel_cnt;
    if (scnt <= kEcCand) {
      if (tid == 0) {
        cand_n = 0;
        cand_sel = INT_MAX;
      }
      __syncthreads();
      each([&](int, float l) {
        if (bucket(l) == sb) {
          const int slot = atomicAdd(&cand_n, 1);
          if (slot < kEcCand) cand_key[slot] = float_key(l);  // (the count is scnt)
        }
      });
      __syncthreads();
      const int n = min(cand_n, kEcCand);
      if (tid < n) {
        const uint32_t kt = cand_key[tid];
        int above = 0, ateq = 0;
        for (int j = 0; j < n; ++j) {
          const uint32_t kj = cand_key[j];
          above += kj > kt;
          ateq += kj >= kt;
        }
        cand_above[tid] = above;
        if (above < sneed && sneed <= ateq) atomicMin(&cand_sel, tid);  // equal keys all hit
      }
      __syncthreads();
      const int cs = cand_sel;  // always set when the bucket's keys are all here
      if (cs < n) {
        prefix = cand_key[cs];
        need = sneed - cand_above[cs];
        found = true;
      }
    }
  }
  // radix select: 8-bit digits of the key from the top
  uint32_t mask = 0;
  for (int shift = 24; shift >= 0 && !found; shift -= 8) {
    for (int i = lane; i < 256; i += 64) whist[wid][i] = 0;
    __builtin_amdgcn_wave_barrier();
    each([&](int, float l) {
      const uint32_t key = float_key(l);
      if ((key & mask) == prefix) atomicAdd(&whist[wid][(key >> shift) & 255u], 1);
    });
    __syncthreads();
    find_bucket(need);
    prefix |= (uint32_t)sel_digit << shift;
    mask |= 255u << shift;
    need = sel_need;
    __syncthreads();
  }
  const uint32_t thr = prefix;  // key of the C-th largest logit
  // `need` = how many keys equal to thr are taken (lowest token indices first)
  // keys above thr and equal to it before this thread (one scan of both counts): every
  // key above is taken, and the first `need` equal ones
  int nabove = 0, neq = 0;
  each([&](int, float l) {
    const uint32_t key = float_key(l);
    nabove += key > thr;
    neq += key == thr;
  });
  long long tot;
  const long long base2 =
      block_exclusive_scan<long long>(((long long)nabove << 32) + neq, scan_sh, &tot);
  const int eq_base = (int)(base2 & 0xffffffffll);
  int out = (int)(base2 >> 32) + min(eq_base, need);
  {
    int eqr = eq_base;
    const int rstride = ec_run_stride(T);
    each([&](int t, float l) {
      // entries before token t: the run table's boundary when t starts a combine block
      if (runs && t % kEcCombineTokens == 0)
        runs[(size_t)e * rstride + t / kEcCombineTokens] = out;
      const uint32_t key = float_key(l);
      bool take = false;
      if (key > thr) take = true;
      else if (key == thr) take = (eqr++ < need);
      const float sc = expf(l - m) / sum;
      if (take && out < C) {
        idx[(size_t)e * C + out] = t;
        if (src) src[(size_t)e * C + out] = t;
        score[(size_t)e * C + out] = sc;
        ++out;
      }
      if (probs) probs[(size_t)t * E + e] = sc;
    });
  }
  if (tid == 0) {
    if (runs) runs[(size_t)e * ec_run_stride(T) + ec_run_stride(T) - 1] = C;
    offsets[e] = e * C;
    if (e == E - 1) offsets[E] = E * C;
    if (counts) counts[e] = C;
  }
}

}  // namespace

hipError_t launch_router(const RouterArgs& a, int bf16in, int ec, hipStream_t s) {
  const int nblk = (a.T + kRT - 1) / kRT;
  const int ep = a.E <= 16 ? 16 : (a.E <= 32 ? 32 : 64);
  const int noise = (a.eps || a.draw) ? (a.Wn ? 2 : 1) : 0;
  if (noise && ec) return hipErrorInvalidValue;  // noise is a token-choice feature
  dim3 grid(nblk), block(256);
  const bool direct = bf16in && a.E % 8 == 0;
#define MOE_ROUTER(TI, EP, NOISE, DIRECT) \
  router_kernel<TI, EP, NOISE, DIRECT><<<grid, block, 0, s>>>(a, ec)
#define MOE_ROUTER_EP(TI, NOISE, DIRECT)                        \
  do {                                                          \
    if (ep == 16) MOE_ROUTER(TI, 16, NOISE, DIRECT);            \
    else if (ep == 32) MOE_ROUTER(TI, 32, NOISE, DIRECT);       \
    else MOE_ROUTER(TI, 64, NOISE, DIRECT);                     \
  } while (0)
  if (bf16in && direct) {
    if (noise == 0) MOE_ROUTER_EP(bf16, 0, true);
    else if (noise == 1) MOE_ROUTER_EP(bf16, 1, true);
    else MOE_ROUTER_EP(bf16, 2, true);
  } else if (bf16in) {
    if (noise == 0) MOE_ROUTER_EP(bf16, 0, false);
    else if (noise == 1) MOE_ROUTER_EP(bf16, 1, false);
    else MOE_ROUTER_EP(bf16, 2, false);
  } else {
    if (noise == 0) MOE_ROUTER_EP(float, 0, false);
    else if (noise == 1) MOE_ROUTER_EP(float, 1, false);
    else MOE_ROUTER_EP(float, 2, false);
  }
#undef MOE_ROUTER_EP
#undef MOE_ROUTER
  return hipGetLastError();
}

hipError_t launch_ec_select(const float* logitsT, int T, int E, int C, int32_t* idx, float* score,
                            float* probs, int32_t* offsets, int32_t* counts, int32_t* src,
                            int32_t* sk_flags, int32_t* runs, hipStream_t s) {
  if (T <= 8 * kEcThreads)
    ec_select_kernel<8><<<E, kEcThreads, 0, s>>>(logitsT, T, E, C, idx, score, probs, offsets,
                                                 counts, src, sk_flags, runs);
  else if (T <= 16 * kEcThreads)
    ec_select_kernel<16><<<E, kEcThreads, 0, s>>>(logitsT, T, E, C, idx, score, probs, offsets,
                                                  counts, src, sk_flags, runs);
  else if (T <= kEcLdsTokens)
    ec_select_kernel<-1><<<E, kEcThreads, 0, s>>>(logitsT, T, E, C, idx, score, probs, offsets,
                                                  counts, src, sk_flags, runs);
  else
    ec_select_kernel<0><<<E, kEcThreads, 0, s>>>(logitsT, T, E, C, idx, score, probs, offsets,
                                                 counts, src, sk_flags, runs);
  return hipGetLastError();
}
