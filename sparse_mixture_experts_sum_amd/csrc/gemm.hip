// Grouped expert GEMMs for gfx950.
//
// Experts are the SwiGLU FFNs of "Mixture of Experts（MoE）の理論と実装" (Expert.forward:
// silu(x W_gate) * (x W1), then W2) and the Korean page's SwiGLUExpert. Rows arrive
// grouped by expert (group e = rows [offsets[e], offsets[e+1])), so each expert's
// rows form one dense GEMM against that expert's weights.
//
// bf16 path (the hot path):
//   * persistent workgroups (one per CU) walk the tile list; each XCD takes a
//     contiguous share of the tiles, in an order that keeps 4 M-tiles x 8 N-tiles of
//     the same weights and rows in flight together, so that XCD's L2 serves the
//     re-reads;
//   * 256 threads, 2x2 waves, v_mfma_f32_32x32x16_bf16 with the weight fragment as
//     the first operand, so that each lane's 16 accumulators are 4 runs of 4
//     consecutive output columns of one row (8- and 16-byte stores);
//   * K steps of 64, double-buffered LDS; the next step's global loads are in flight
//     while the current step's MFMAs run;
//   * weights are stored [K, N] (the x @ W layout of the pages), N contiguous; each
//     thread loads an 8x8 block (8 rows of 16 bytes) and transposes it in registers
//     so that LDS holds K-contiguous rows, which the MFMA operand needs;
//   * gate and up tiles share the A tile; the SwiGLU epilogue silu(g) * u runs in
//     registers and writes h in bf16. The down projection writes o in fp32.
//
// fp32 path: a plain LDS-tiled FMA kernel (64x64 tiles, 4x4 outputs per thread).
#include "common.h"
#include "kernels.h"

namespace {

constexpr int BK = 64;
constexpr int kGroupM = 4;  // M-tiles walked together per group of N-tiles

// LDS tile rows are 64 bf16 = 8 chunks of 16 bytes; chunks are XOR-swizzled so that
// the MFMA fragment reads (32 rows, same chunk) and the stores hit distinct banks.
__device__ __forceinline__ int a_off(int row, int c) { return row * 64 + ((c ^ (row & 7)) << 3); }
__device__ __forceinline__ int b_off(int n, int c) {
  return n * 64 + ((c ^ ((n + (n >> 3)) & 7)) << 3);
}

// 8 rows (k) x 8 bf16 (n) in, 8 columns x 8 bf16 (k) out.
__device__ __forceinline__ void transpose8x8(const u32x4 (&r)[8], u32x4 (&c)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t lo = r[2 * m][j >> 1], hi = r[2 * m + 1][j >> 1];
      c[j][m] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
}

__device__ __forceinline__ int count_mtiles(const int32_t* offsets, int E, int BM) {
  int mt = 0;
  for (int e = 0; e < E; ++e) mt += (offsets[e + 1] - offsets[e] + BM - 1) / BM;
  return mt;
}

// Expert owning M-tile `mt`, and that tile's first row and row count.
__device__ __forceinline__ void locate_mtile(const int32_t* offsets, int BM, int mt, int& e,
                                             int& row0, int& rows) {
  int acc = 0;
  e = 0;
  for (;;) {
    const int ne = offsets[e + 1] - offsets[e];
    const int te = (ne + BM - 1) / BM;
    if (mt < acc + te) break;
    acc += te;
    ++e;
  }
  row0 = offsets[e] + (mt - acc) * BM;
  rows = min(BM, offsets[e + 1] - row0);
}

template <int BM, int BN, bool SWIGLU>
struct Cfg {
  static constexpr int NBL = SWIGLU ? 2 * BN : BN;  // weight columns staged per tile
  static constexpr int WM = BM / 2, WN = BN / 2;    // per wave (2 x 2 waves)
  static constexpr int MB = WM / 32, NB = WN / 32;  // 32x32 blocks per wave
  static constexpr int NMAT = SWIGLU ? 2 : 1;
  static constexpr int A_PER = BM * 8 / 256;        // 16-byte A chunks per thread per K step
  static constexpr int B_PER = (NBL + 255) / 256;   // 8x8 weight blocks per thread per K step
  static constexpr int LDS_A = BM * BK, LDS_B = NBL * BK;
  static constexpr int STAGE = LDS_A + LDS_B;
  static_assert(MB >= 1 && NB >= 1, "tile too small for 2x2 waves of 32x32 blocks");
};

template <int BM, int BN, bool SWIGLU>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_bf16_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ B0, const bf16* __restrict__ B1,
    const int32_t* __restrict__ offsets, int E, int K, int N, void* __restrict__ out) {
  using C = Cfg<BM, BN, SWIGLU>;
  extern __shared__ __attribute__((aligned(16))) bf16 lds[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const int MT = count_mtiles(offsets, E, BM);
  const int NT = N / BN;
  const int total = MT * NT;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, nslot = gridDim.x >> 3;
  const int lo = (int)(((long long)total * xcd) >> 3);
  const int hi = (int)(((long long)total * (xcd + 1)) >> 3);
  const int nk = K / BK;

  for (int tile = lo + slot; tile < hi; tile += nslot) {
    const int grp = tile / (kGroupM * NT);
    const int m_first = grp * kGroupM;
    const int gm = min(kGroupM, MT - m_first);
    const int rem = tile - grp * kGroupM * NT;
    const int nt = rem / gm, mt = m_first + rem % gm;
    int e, row0, rows;
    locate_mtile(offsets, BM, mt, e, row0, rows);
    const int n0 = nt * BN;

    const bf16* Ab = A + (size_t)row0 * K;
    const bf16* W0 = B0 + (size_t)e * K * N;
    const bf16* W1 = SWIGLU ? B1 + (size_t)e * K * N : nullptr;

    // global -> register staging
    u32x4 ra[C::A_PER];
    u32x4 rb[C::B_PER][8];
    // element offsets from Ab (rows past the group's end re-read its last row)
    int a_src[C::A_PER];
#pragma unroll
    for (int i = 0; i < C::A_PER; ++i) {
      const int r = (tid >> 3) + 32 * i;
      a_src[i] = min(r, rows - 1) * K + (tid & 7) * 8;
    }
    const bf16* b_src[C::B_PER];
    int b_nl[C::B_PER], b_kg[C::B_PER];
#pragma unroll
    for (int j = 0; j < C::B_PER; ++j) {
      const int bid = tid + 256 * j;
      const int ng = bid % (C::NBL / 8), kg = bid / (C::NBL / 8);
      const int nl = 8 * ng;
      b_nl[j] = nl;
      b_kg[j] = kg;
      const bf16* W = (SWIGLU && nl >= BN) ? W1 : W0;
      const int ncol = n0 + ((SWIGLU && nl >= BN) ? nl - BN : nl);
      b_src[j] = W + (size_t)(8 * kg) * N + ncol;
    }
    auto gload = [&](int kt) {
      const size_t koff = (size_t)kt * BK;
#pragma unroll
      for (int i = 0; i < C::A_PER; ++i) ra[i] = ld16(Ab + koff + a_src[i]);
#pragma unroll
      for (int j = 0; j < C::B_PER; ++j) {
        if (tid + 256 * j < C::NBL) {
#pragma unroll
          for (int q = 0; q < 8; ++q) rb[j][q] = ld16(b_src[j] + (koff + q) * N);
        }
      }
    };
    auto sstore = [&](int stage) {
      bf16* As = lds + stage * C::STAGE;
      bf16* Bs = As + C::LDS_A;
#pragma unroll
      for (int i = 0; i < C::A_PER; ++i) st16(As + a_off((tid >> 3) + 32 * i, tid & 7), ra[i]);
#pragma unroll
      for (int j = 0; j < C::B_PER; ++j) {
        if (tid + 256 * j < C::NBL) {
          u32x4 col[8];
          transpose8x8(rb[j], col);
#pragma unroll
          for (int q = 0; q < 8; ++q) st16(Bs + b_off(b_nl[j] + q, b_kg[j]), col[q]);
        }
      }
    };

    f32x16 acc[C::NMAT][C::NB][C::MB];
#pragma unroll
    for (int mt_ = 0; mt_ < C::NMAT; ++mt_)
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[mt_][nb][mb][r] = 0.f;

    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) gload(kt + 1);
      const bf16* As = lds + cur * C::STAGE;
      const bf16* Bs = As + C::LDS_A;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int cc = 2 * s + (lane >> 5);
        bf16x8 af[C::MB];
        bf16x8 bfr[C::NMAT][C::NB];
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
          const int m = wm * C::WM + mb * 32 + (lane & 31);
          af[mb] = __builtin_bit_cast(bf16x8, ld16(As + a_off(m, cc)));
        }
#pragma unroll
        for (int mt_ = 0; mt_ < C::NMAT; ++mt_)
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb) {
            const int n = mt_ * BN + wn * C::WN + nb * 32 + (lane & 31);
            bfr[mt_][nb] = __builtin_bit_cast(bf16x8, ld16(Bs + b_off(n, cc)));
          }
#pragma unroll
        for (int mt_ = 0; mt_ < C::NMAT; ++mt_)
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
            for (int mb = 0; mb < C::MB; ++mb)
              acc[mt_][nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  bfr[mt_][nb], af[mb], acc[mt_][nb][mb], 0, 0, 0);
      }
      if (kt + 1 < nk) sstore(cur ^ 1);
      __syncthreads();
    }

    // epilogue: acc[.][nb][mb][4q + i] = out[row = m][col = n0 + ncol0 + 8q + 4*(lane/32) + i]
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        const int m = wm * C::WM + mb * 32 + (lane & 31);
        if (m >= rows) continue;
        const size_t rowoff = (size_t)(row0 + m) * N + n0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ncol = wn * C::WN + nb * 32 + 8 * q + 4 * (lane >> 5);
          if constexpr (SWIGLU) {
            bf16x4 hv;
#pragma unroll
            for (int i = 0; i < 4; ++i)
              hv[i] = (bf16)(silu(acc[0][nb][mb][4 * q + i]) * acc[1][nb][mb][4 * q + i]);
            *reinterpret_cast<u32x2*>(static_cast<bf16*>(out) + rowoff + ncol) =
                __builtin_bit_cast(u32x2, hv);
          } else {
            f32x4 v = {acc[0][nb][mb][4 * q + 0], acc[0][nb][mb][4 * q + 1],
                       acc[0][nb][mb][4 * q + 2], acc[0][nb][mb][4 * q + 3]};
            *reinterpret_cast<f32x4*>(static_cast<float*>(out) + rowoff + ncol) = v;
          }
        }
      }
  }
}

// ---------------------------------------------------------------------------------
// fp32: 64x64 output tiles, K steps of 16, 16x16 threads with 4x4 outputs each.
// ---------------------------------------------------------------------------------
template <bool SWIGLU>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A,
                                                       const float* __restrict__ B0,
                                                       const float* __restrict__ B1,
                                                       const int32_t* __restrict__ offsets, int E,
                                                       int K, int N, float* __restrict__ out) {
  constexpr int TM = 64, TN = 64, TK = 16;
  __shared__ float As[TK][TM + 4];
  __shared__ float Bs[SWIGLU ? 2 : 1][TK][TN];
  const int MT = count_mtiles(offsets, E, TM);
  const int mt = blockIdx.y;
  if (mt >= MT) return;
  int e, row0, rows;
  locate_mtile(offsets, TM, mt, e, row0, rows);
  const int n0 = blockIdx.x * TN;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const float* W0 = B0 + (size_t)e * K * N;
  const float* W1 = SWIGLU ? B1 + (size_t)e * K * N : nullptr;
  float acc[2][4][4] = {};
  const int ar = tid >> 2, ak = (tid & 3) * 4;
  const float* arow = A + (size_t)(row0 + min(ar, rows - 1)) * K;
  const int bk = tid >> 4, bn = (tid & 15) * 4;
  for (int k0 = 0; k0 < K; k0 += TK) {
    const f32x4 av = *reinterpret_cast<const f32x4*>(arow + k0 + ak);
#pragma unroll
    for (int i = 0; i < 4; ++i) As[ak + i][ar] = av[i];
    *reinterpret_cast<f32x4*>(&Bs[0][bk][bn]) =
        *reinterpret_cast<const f32x4*>(W0 + (size_t)(k0 + bk) * N + n0 + bn);
    if constexpr (SWIGLU)
      *reinterpret_cast<f32x4*>(&Bs[1][bk][bn]) =
          *reinterpret_cast<const f32x4*>(W1 + (size_t)(k0 + bk) * N + n0 + bn);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&As[kk][ty * 4]);
#pragma unroll
      for (int m = 0; m < (SWIGLU ? 2 : 1); ++m) {
        const f32x4 b = *reinterpret_cast<const f32x4*>(&Bs[m][kk][tx * 4]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[m][i][j] = fmaf(a[i], b[j], acc[m][i][j]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = ty * 4 + i;
    if (m >= rows) continue;
    f32x4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = SWIGLU ? silu(acc[0][i][j]) * acc[1][i][j] : acc[0][i][j];
    *reinterpret_cast<f32x4*>(out + (size_t)(row0 + m) * N + n0 + tx * 4) = v;
  }
}

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

template <int BM, int BN, bool SWIGLU>
hipError_t launch_bf16(const void* A, const void* B0, const void* B1, const int32_t* offsets, int E,
                       int K, int N, void* out, hipStream_t s) {
  using C = Cfg<BM, BN, SWIGLU>;
  const size_t lds_bytes = 2 * C::STAGE * sizeof(bf16);
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t err = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemm_bf16_kernel<BM, BN, SWIGLU>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    if (err != hipSuccess) return err;
    attr_done = true;
  }
  const int grid = ((device_cu_count() + 7) / 8) * 8;
  gemm_bf16_kernel<BM, BN, SWIGLU><<<grid, 256, lds_bytes, s>>>(
      static_cast<const bf16*>(A), static_cast<const bf16*>(B0), static_cast<const bf16*>(B1),
      offsets, E, K, N, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_gateup(int bf16in, const void* xp, const void* Wgate, const void* Wup,
                              const int32_t* offsets, int E, int R_max, int d, int f, void* h,
                              hipStream_t s) {
  if (bf16in) {
    if (f % 128 == 0) return launch_bf16<256, 128, true>(xp, Wgate, Wup, offsets, E, d, f, h, s);
    return launch_bf16<256, 64, true>(xp, Wgate, Wup, offsets, E, d, f, h, s);
  }
  dim3 grid(f / 64, R_max / 64 + E);
  gemm_f32_kernel<true><<<grid, 256, 0, s>>>(static_cast<const float*>(xp),
                                             static_cast<const float*>(Wgate),
                                             static_cast<const float*>(Wup), offsets, E, d, f,
                                             static_cast<float*>(h));
  return hipGetLastError();
}

hipError_t launch_gemm_down(int bf16in, const void* h, const void* Wdown, const int32_t* offsets,
                            int E, int R_max, int f, int d, float* o, hipStream_t s) {
  if (bf16in) {
    if (d % 256 == 0) return launch_bf16<256, 256, false>(h, Wdown, nullptr, offsets, E, f, d, o, s);
    if (d % 128 == 0) return launch_bf16<256, 128, false>(h, Wdown, nullptr, offsets, E, f, d, o, s);
    return launch_bf16<256, 64, false>(h, Wdown, nullptr, offsets, E, f, d, o, s);
  }
  dim3 grid(d / 64, R_max / 64 + E);
  gemm_f32_kernel<false><<<grid, 256, 0, s>>>(static_cast<const float*>(h),
                                              static_cast<const float*>(Wdown), nullptr, offsets,
                                              E, f, d, o);
  return hipGetLastError();
}
