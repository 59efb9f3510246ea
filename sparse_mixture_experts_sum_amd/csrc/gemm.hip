// Grouped expert GEMMs for gfx950.
//
// Experts are the SwiGLU FFNs of "Mixture of Experts（MoE）の理論と実装" (Expert.forward:
// silu(x W_gate) * (x W1), then W2) and the Korean page's SwiGLUExpert. Rows arrive
// grouped by expert (group e = rows [offsets[e], offsets[e+1])), so each expert's
// rows form one dense GEMM against that expert's weights.
//
// bf16 path (the hot path):
//   * persistent workgroups (one per CU); all XCDs walk the experts in the same order,
//     XCD x owning the x-th eighth of each expert's output columns and walking them in
//     blocks of a few columns, so that an XCD's concurrent tiles share both their rows
//     and their weight columns in its L2 and the XCDs share the expert's rows in the
//     memory-side cache; when every expert has few tiles, each XCD takes a contiguous
//     run of experts instead (TileMap);
//   * v_mfma_f32_32x32x16_bf16 with the weight fragment as the first operand, so that
//     each lane's 16 accumulators are 4 runs of 4 consecutive output columns of one row
//     (8- and 16-byte stores);
//   * K stages of 32 through a ring of 4 LDS buffers filled by direct global->LDS loads
//     (no registers in between); weights stay [K, N] as the pages store them and the B
//     fragments come out of LDS with ds_read_b64_tr_b16 (transposing reads), the A
//     fragments with 16-byte reads; both layouts are swizzled so that the fragment reads
//     are free of bank conflicts;
//   * 256 x 256 tiles: four waves (one per SIMD), each a 128 x 128 block with its 256
//     accumulators in AGPRs, software-pipelined (PipeStep): the MFMAs of one stage run
//     while the fragments of the next are read and the ring is refilled, one barrier
//     per stage, and the stages stream across tiles (pipe_stream). Smaller tiles
//     (256 x 128, 256 x 64) use the plain ring (ring_step);
//   * gate and up tiles share the A tile; the SwiGLU epilogue silu(g) * u runs in
//     registers and writes h in bf16 (plus its bf16 residual when asked: SPLIT). The
//     down projection writes o in fp32; with SPLIT it runs h and its residual as pairs:
//     a 256-row tile holds 128 tokens' main and residual rows, and the epilogue adds the
//     two products of each token before its single store.
//
// fp32 path: a plain LDS-tiled FMA kernel (64x64 tiles, 4x4 outputs per thread).
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kBK = 32;       // K per LDS stage
constexpr int kStages = 4;    // LDS ring stages; kStages - 1 are in flight

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

// silu(z) = z * sigmoid(z) from the hardware base-2 exponential and reciprocal (about
// 1 ulp each). The bf16 path rounds h to 8 significant bits (or keeps a 16-bit pair),
// far coarser than these; the IEEE division and range-reduced expf would cost about
// four times the VALU work in an epilogue that no other wave hides at one wave per SIMD.
// Limits: z -> +inf gives z; z -> -inf gives exp2 = inf, reciprocal 0, result -0.
__device__ __forceinline__ float silu_bf16_path(float z) {
  const float e = __builtin_amdgcn_exp2f(z * -1.4426950408889634f);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// s_waitcnt lgkmcnt(0): this wave's LDS reads have returned
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14)); }

// Workgroup barrier that the instruction scheduler does not move code across.
__device__ __forceinline__ void sync_point() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Tile geometry. BM rows x BNL staged weight columns per tile (SwiGLU: BNL/2 gate
// columns then BNL/2 up columns, BNL/2 outputs), K staged in steps of 32 through a
// ring of 4 LDS stages filled by direct global->LDS loads (each wave instruction
// moves 64 lanes x 16 bytes into 1 KB of LDS, lane l into slot l).
//
// LDS layouts (per stage):
//   A [BM][32] bf16, 64-byte rows, 16-byte chunk c stored at c ^ ((row >> 1) & 3)
//   B [32][BNL] bf16 (k rows, n contiguous, as the weights sit in HBM), 16-byte slot
//     s of row k stored at s ^ (2 * (k & 3))
// MFMA operands: the A fragment is one 16-byte LDS read per lane (8 consecutive k of
// one row); the B fragment is two ds_read_b64_tr_b16 per lane, each of which hands
// every lane of a 16-lane group 4 consecutive k of one column: source lane i of the
// group addresses row k0 + i/4, columns n0 + 4*(i%4) .. +3, and result lane j gets
// element j%4 of source lanes j/4, j/4 + 4, j/4 + 8, j/4 + 12.
// 16-byte chunk swizzles (see the layout notes above): conflict-free fragment reads for
// 32- and 64-bank LDS. A rows hold CPR chunks (4 for K stages of 32, 8 for 64).
template <int CPR>
__device__ __forceinline__ int a_swz(int row) {
  if constexpr (CPR == 4) return ((row >> 1) ^ (row >> 3)) & 3;
  else return (row ^ (row >> 3)) & 7;
}
__device__ __forceinline__ int b_swz(int k) { return (0xCA60 >> (4 * (k & 3))) & 15; }  // 0,6,10,12

template <int BM, int BNL, bool SWIGLU, bool SPLIT, int NW>
struct Geo {
  static constexpr int BK = kBK, STAGES = kStages;
  static constexpr int SUB = BK / 16;                // 16-deep MFMA substeps per stage
  static constexpr int A_CPR = BK / 8;               // 16-byte chunks per A row
  static constexpr int A_RPI = 1024 / (BK * 2);      // A rows per DMA instruction
  static constexpr bool GATHERS = SWIGLU;             // A rows may be gathered (gate/up)
  static constexpr int WGN = NW / 2;                 // waves: 2 along M x WGN along N
  static constexpr int WM = BM / 2, WNL = BNL / WGN; // per wave
  static constexpr int MB = WM / 32, NBW = WNL / 32; // 32x32 blocks per wave
  static constexpr int BN_OUT = SWIGLU ? BNL / 2 : BNL;
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * BNL * 2;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int A_PW = A_BYTES / 1024 / NW;   // DMA instructions per wave per stage
  static constexpr int B_PW = B_BYTES / 1024 / NW;
  static constexpr int LPS = A_PW + B_PW;            // loads per wave per stage
  static constexpr int B_ROW = BNL * 2;              // bytes per B row
  static constexpr int B_SLOTS = BNL / 8;
  static constexpr int B_RPI = 1024 / B_ROW;         // B rows per DMA instruction
  static_assert(MB >= 1 && NBW >= 1 && (!SWIGLU || NBW % 2 == 0), "tile shape");
  static_assert(A_PW >= 1 && B_PW >= 1, "tile too small for the waves' DMA");
  static constexpr size_t LDS = (size_t)STAGES * STAGE_BYTES;
};

// Direct loads of one K stage of the A and B tiles into a ring buffer.
template <class G, bool SWIGLU, bool SPLIT>
struct StageLoader {
  const bf16* Ab;                 // A rows of this tile (h or x_perm)
  const bf16* b_base[G::B_PW];    // weight matrix each B instruction reads
  int a_src[G::A_PW];             // per-lane element offsets (row, chunk)
  int b_src[G::B_PW];
  int nk, N, wave;

  // load j (0 .. LPS-1: A loads, then B loads; a constant at every call) of stage kt
  // into stage buffer st
  __device__ __forceinline__ void issue_one(int j, int kt, char* st) const {
    const int kk = kt * G::BK;
    if (j < G::A_PW) {
      __builtin_amdgcn_global_load_lds(Ab + kk + a_src[j],
                                       (lds_void*)(st + (wave * G::A_PW + j) * 1024), 16, 0, 0);
    } else {
      const int jb = j - G::A_PW;
      __builtin_amdgcn_global_load_lds(b_base[jb] + (size_t)kk * N + b_src[jb],
                                       (lds_void*)(st + G::A_BYTES + (wave * G::B_PW + jb) * 1024),
                                       16, 0, 0);
    }
  }
  __device__ __forceinline__ void issue(int kt, char* st) const {
    const int kk = kt * G::BK;
#pragma unroll
    for (int j = 0; j < G::A_PW; ++j)
      __builtin_amdgcn_global_load_lds(Ab + kk + a_src[j],
                                       (lds_void*)(st + (wave * G::A_PW + j) * 1024), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < G::B_PW; ++j)
      __builtin_amdgcn_global_load_lds(b_base[j] + (size_t)kk * N + b_src[j],
                                       (lds_void*)(st + G::A_BYTES + (wave * G::B_PW + j) * 1024),
                                       16, 0, 0);
  }
};

// min(max(n, 0), 2): stages that may stay in flight after the one waited for
__device__ __forceinline__ int clamp_stages(int n) { return n < 0 ? 0 : (n > 2 ? 2 : n); }

// s_waitcnt vmcnt(n * PER) for a runtime n in [0, 3]
template <int PER>
__device__ __forceinline__ void wait_stages(int n) {
  if (n >= 3) wait_vmcnt<3 * PER>();
  else if (n == 2) wait_vmcnt<2 * PER>();
  else if (n == 1) wait_vmcnt<PER>();
  else wait_vmcnt<0>();
}

// One K stage: wait for stage kt's loads, barrier, refill the ring STAGES - 1 stages
// ahead, then SUB x (fragment reads + MB x NBW MFMAs). J = kt % STAGES is a template
// argument so that every LDS access names one of the stage arrays; FULL steps always
// refill, so that the compiler sees the same number of loads in flight on every path.
// (TAG: see k_loop)
template <class G, bool SWIGLU, bool SPLIT, int J, bool FULL, int TAG>
__device__ __forceinline__ void ring_step(int kt, int nk_total, char* const (&ring)[G::STAGES],
                                          const StageLoader<G, SWIGLU, SPLIT>& ld,
                                          const int (&a_frag)[G::MB], const int (&b_frag)[G::NBW],
                                          f32x16 (&acc)[G::NBW][G::MB]) {
  constexpr int AHEAD = G::STAGES - 1;
  static_assert(AHEAD >= 1 && AHEAD <= 3, "ring depth");
  // this wave's loads for stage kt have landed (later stages may still be in flight)
  if constexpr (FULL) wait_vmcnt<(AHEAD - 1) * G::LPS>();
  else wait_stages<G::LPS>(min(AHEAD - 1, nk_total - 1 - kt));
  // everyone's loads for stage kt have landed, and everyone is done with stage kt-1
  __builtin_amdgcn_s_barrier();
  if (FULL || kt + AHEAD < nk_total) ld.issue(kt + AHEAD, ring[(J + AHEAD) % G::STAGES]);
  const char* st = ring[J];
#pragma unroll
  for (int s = 0; s < G::SUB; ++s) {
    bf16x8 af[G::MB], bfr[G::NBW];
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
      af[mb] = *reinterpret_cast<const bf16x8*>(st + (a_frag[mb] ^ (32 * s)));
#pragma unroll
    for (int nb = 0; nb < G::NBW; ++nb) {
      const char* bp = st + b_frag[nb] + 16 * s * G::B_ROW;
      const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)bp);
      const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(bp + 4 * G::B_ROW));
      const s16x8 v = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      bfr[nb] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int nb = 0; nb < G::NBW; ++nb)
#pragma unroll
      for (int mb = 0; mb < G::MB; ++mb)
        acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[nb], af[mb], acc[nb][mb], 0, 0, 0);
    // keep the scheduler from hoisting more than two substeps' fragment reads (register
    // pressure) when a stage holds more than 32 of K
    if (s % 2 == 1 && s + 1 < G::SUB) __builtin_amdgcn_sched_barrier(0);
  }
}

// Fragments of one K stage for one wave: A as SUB x MB 8-element rows, B as the two
// transposed 4-element halves of SUB x NBW fragments.
template <class G>
struct Frags {
  bf16x8 a[G::SUB][G::MB];
  s16x4 blo[G::SUB][G::NBW], bhi[G::SUB][G::NBW];
};

// LDS read r of a stage's fragments (r constant at every call): first the SUB x MB A
// rows, then for each (substep, block) the two halves of the B fragment.
template <class G>
__device__ __forceinline__ void read_frag(int r, const char* st, const int (&a_frag)[G::MB],
                                          const int (&b_frag)[G::NBW], Frags<G>& F) {
  constexpr int NA = G::SUB * G::MB;
  if (r < NA) {
    const int s = r / G::MB, mb = r % G::MB;
    F.a[s][mb] = *reinterpret_cast<const bf16x8*>(st + (a_frag[mb] ^ (32 * s)));
  } else {
    const int i = r - NA, s = i / (2 * G::NBW), nb = (i / 2) % G::NBW, h = i % 2;
    const char* bp = st + b_frag[nb] + 16 * s * G::B_ROW + h * 4 * G::B_ROW;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)bp);
    if (h) F.bhi[s][nb] = v;
    else F.blo[s][nb] = v;
  }
}

template <class G>
__device__ __forceinline__ void mfma_frag(int i, const Frags<G>& F, f32x16 (&acc)[G::NBW][G::MB]) {
  const int s = i / (G::NBW * G::MB), nb = i / G::MB % G::NBW, mb = i % G::MB;
  const s16x4 lo = F.blo[s][nb], hi = F.bhi[s][nb];
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v), F.a[s][mb],
                                                        acc[nb][mb], 0, 0, 0);
}

// Software-pipelined K stage for one wave per SIMD (fragments double-buffered in
// registers). Step kt: wait for the own loads of stage kt+1 and for the own LDS reads of
// stage kt, barrier; then the MFMAs of stage kt (fragments read in the previous step)
// with, spread between them, the LDS reads of stage kt+1 and the refill of stage kt's
// buffer with stage kt+STAGES. Correctness: every wave's loads of stage kt+1 have landed
// before any wave reads it (each waits before the barrier), and every wave's reads of
// stage kt are complete (lgkmcnt(0) before the barrier) before any wave refills its
// buffer after the barrier.
// FULL steps read the next stage and refill; otherwise `more` and `refill` say which
// happens and n_after is the number of stages in flight after the next one. The refill
// loads stage `rstage` of loader `rl` (the next tile's loader near the end of a tile).
// (A class template: hipcc's host pass rejects later calls of this step as a function
// template once it has been instantiated from two callers.)
template <class G, bool SWIGLU, bool SPLIT, int J, bool FULL>
struct PipeStep {
static __device__ __forceinline__ void run(int n_after, bool more_, bool refill_,
                                          const StageLoader<G, SWIGLU, SPLIT>& rl, int rstage,
                                          char* const (&ring)[G::STAGES],
                                          const int (&a_frag)[G::MB], const int (&b_frag)[G::NBW],
                                          f32x16 (&acc)[G::NBW][G::MB], const Frags<G>& Fc,
                                          Frags<G>& Fn) {
  constexpr int S = G::STAGES;
  constexpr int NM = G::SUB * G::NBW * G::MB;                // MFMAs per stage
  constexpr int NR = G::SUB * G::MB + 2 * G::SUB * G::NBW;   // LDS reads per stage
  constexpr int NG = G::LPS;                                 // groups: one load each
  static_assert(NM >= NG && NR >= NG, "MFMA / read / load groups");
  __builtin_amdgcn_sched_barrier(0);
  // own loads of stage kt + 1 (kt + 1 .. kt + S - 1 may be in flight)
  if constexpr (FULL) wait_vmcnt<(S - 2) * G::LPS>();
  else wait_stages<G::LPS>(n_after);
  wait_lgkmcnt0();
  sync_point();
  const bool more = FULL || more_;
  const bool refill = FULL || refill_;
  const char* src = ring[(J + 1) % S];
  char* const dst = ring[J];
  // group g: MFMAs [NM g / NG, NM (g + 1) / NG), reads likewise, then one load (equal
  // groups when the counts divide)
#pragma unroll
  for (int g = 0; g < NG; ++g) {
#pragma unroll
    for (int m = NM * g / NG; m < NM * (g + 1) / NG; ++m) mfma_frag<G>(m, Fc, acc);
    if (more) {
#pragma unroll
      for (int r = NR * g / NG; r < NR * (g + 1) / NG; ++r)
        read_frag<G>(r, src, a_frag, b_frag, Fn);
    }
    if (refill) rl.issue_one(g, rstage, dst);
    __builtin_amdgcn_sched_barrier(0);
  }
}
};

// The K loop of one tile through the plain ring (ring_step).
// (TAG separates the instantiations of different kernels: hipcc's host pass rejects a
// second call of a function template with these array-reference parameters from
// another kernel with the same arguments)
template <class G, bool SWIGLU, bool SPLIT, int TAG>
__device__ __forceinline__ void k_loop(int nk_total, char* const (&ring)[G::STAGES],
                                       const StageLoader<G, SWIGLU, SPLIT>& ld,
                                       const int (&a_frag)[G::MB], const int (&b_frag)[G::NBW],
                                       f32x16 (&acc)[G::NBW][G::MB]) {
  constexpr int S = G::STAGES;
  int kt = 0;
#define MOE_STEP(J, FULL, KT) \
  ring_step<G, SWIGLU, SPLIT, J, FULL, TAG>(KT, nk_total, ring, ld, a_frag, b_frag, acc)
  // Prologue: stages 0 .. S-2 in flight. The main loop (every step refills) sits in the
  // same branch as an unconditional prologue, so that the compiler sees the same loads
  // in flight on every path into it. At most 2 * S - 2 stages remain after it.
  if (nk_total >= 2 * S - 1) {
#pragma unroll
    for (int i = 0; i < S - 1; ++i) ld.issue(i, ring[i]);
    for (; kt + 2 * S - 1 <= nk_total; kt += S) {
      MOE_STEP(0, true, kt);
      MOE_STEP(1, true, kt + 1);
      if constexpr (S > 2) { MOE_STEP(2 % S, true, kt + 2); }
      if constexpr (S > 3) { MOE_STEP(3 % S, true, kt + 3); }
    }
  } else {
#pragma unroll
    for (int i = 0; i < S - 1; ++i)
      if (i < nk_total) ld.issue(i, ring[i]);
  }
  if (kt < nk_total) { MOE_STEP(0, false, kt); }
  if (kt + 1 < nk_total) { MOE_STEP(1 % S, false, kt + 1); }
  if constexpr (S > 2) {
    if (kt + 2 < nk_total) { MOE_STEP(2 % S, false, kt + 2); }
    if (kt + 3 < nk_total) { MOE_STEP(3 % S, false, kt + 3); }
  }
  if constexpr (S > 3) {
    if (kt + 4 < nk_total) { MOE_STEP(4 % S, false, kt + 4); }
    if (kt + 5 < nk_total) { MOE_STEP(5 % S, false, kt + 5); }
  }
#undef MOE_STEP
}

// Kernel arguments shared by the tile helpers.
struct GemmArgs {
  const bf16* A;         // rows (x, x_perm or h), [*, K]
  const int32_t* gather; // row r of the grouped problem is row gather[r] of A; nullptr: row r
  const bf16* B0;        // W_gate or W_down, [E, K, N]
  const bf16* B1;        // W_up (SwiGLU)
  const int32_t* offsets;
  int E, K, N;
  void* out;             // h (bf16) or o (fp32)
  void* out2;            // h_lo (bf16, SPLIT): the bf16 rounding residual of h
  float* partial;        // stream-K partial sums, one slot per workgroup (nullptr: no stream-K)
  int32_t* flags;        // stream-K: flags[slot] = 1 once that slot's partial is written
  int lo_rows;           // paired down projection (SPLIT): each main row's residual row sits
                         // lo_rows rows after it in A
};

// One output tile: expert e, rows [row0, row0 + rows), output columns from n0.
struct TileCoord {
  int e, row0, rows, n0;
};

// How the tiles are dealt to the eight XCDs (each XCD runs 32 at a time, one per CU).
//  - Columns (groups with many tiles, N-tiles a multiple of 8): the groups are processed one
//    after another by all XCDs together. The XCDs form RP row groups x 8 / RP column groups
//    (RP = 1 or 2): XCD x owns the (x % (8 / RP))-th column group's share of each group's
//    output columns (NX = NT * RP / 8 N-tiles) for the row tiles r of the group with
//    r % RP = (x / (8 / RP) + e) % RP, and walks that rectangle in column blocks of GN
//    N-tiles, rows outer and the block's columns inner. The 32 tiles an XCD runs together
//    then cover about 32 / GN row tiles x GN column tiles, so they share both their rows and
//    their weight columns in the XCD's L2 (about 32 / GN + GN tile operands fetched per 32
//    tiles, against 33 for one column of 32 row tiles). Over the whole launch every row tile
//    is fetched by the 8 / RP XCDs of its row group and every weight column by RP XCDs: the
//    launch picks RP = 2 where that fetches less (rows and weights of about the same size).
//  - Split (groups with many tiles, N-tiles not a multiple of 8; tiles listed
//    N-tile-major): XCD x takes the x-th eighth of each group's list, i.e. mostly its own
//    slice of the group's weight columns, for all of the group's rows.
//  - Contiguous (every group small: the split order would give each XCD under 4 tiles of a
//    group, the columns order under 2, or under 6 when the rows are gathered from x): the
//    groups' lists are concatenated and XCD x takes the x-th eighth of the whole list. The tiles an XCD runs together then come from one or a few
//    groups and share their weight columns and rows in the XCD's L2; split, they would
//    come from a different group each. (Measured: contiguous gains where split leaves
//    an XCD up to 2-3 tiles per group (mid-size down projection, A/B in one process:
//    107.6 -> 102.5 us), and on gathered rows up to about 6 per group; against the columns
//    order at 2-3 tiles per group (64-expert down projection) it was level, and beyond 6
//    with gathered rows split was faster.)
// Both keep the XCDs' tile counts within one of each other.
constexpr int kXcds = 8;
constexpr int kContigTiles = 16;        // max tiles per group for contiguous, plain rows
constexpr int kContigSplitTiles = 32;   // the same where the columns order does not apply
constexpr int kContigGatherTiles = 48;  // the same, rows gathered from x
struct TileMap {
  int NT, xcd, E;
  bool contiguous;
  int base;      // contiguous: this XCD's first tile in the whole list
  int my_total;  // tiles of this XCD
  int nx, gn;    // columns order: N-tiles per XCD and per column block (gn = 0: split order)
};

// Row tiles r < mte with r % rp = s: this XCD's share of a group in the columns order.
__device__ __forceinline__ int row_share(int mte, int rp, int s) {
  return mte > s ? (mte - 1 - s) / rp + 1 : 0;
}

// CONTIG_OK: the shape allows the contiguous order (a group of one M-tile has NT tiles,
// so NT at or above the threshold rules it out; the launch picks the instantiation).
template <int BM, bool CONTIG_OK, int RP>
__device__ __forceinline__ TileMap make_tile_map(const int32_t* offsets, int E, int NT, int xcd,
                                                 bool gathered, int gn) {
  constexpr int rp = RP;
  TileMap m;
  m.NT = NT;
  m.xcd = xcd;
  m.E = E;
  m.nx = NT / (kXcds / rp);
  m.gn = gn;
  long long total = 0, maxpe = 0;
  int split_total = 0, col_total = 0;
  for (int e = 0; e < E; ++e) {
    const int mte = (offsets[e + 1] - offsets[e] + BM - 1) / BM;
    const long long pe = (long long)mte * NT;
    if constexpr (CONTIG_OK) {
      total += pe;
      maxpe = pe > maxpe ? pe : maxpe;
    }
    split_total += (int)((pe * (xcd + 1)) >> 3) - (int)((pe * xcd) >> 3);
    if constexpr (RP == 1) col_total += mte * m.nx;
    else col_total += row_share(mte, RP, (xcd / (kXcds / RP) + e) % RP) * m.nx;
  }
  // (contiguous: every group has fewer than 48 tiles, so the whole list fits an int)
  m.contiguous = CONTIG_OK && maxpe < (gathered ? kContigGatherTiles
                                                : (gn > 0 ? kContigTiles : kContigSplitTiles));
  if (m.contiguous) m.gn = 0;
  m.base = m.contiguous ? (int)((total * xcd) >> 3) : 0;
  m.my_total = m.contiguous ? (int)((total * (xcd + 1)) >> 3) - m.base
                            : (m.gn > 0 ? col_total : split_total);
  return m;
}

// Where a workgroup stands in its XCD's tile list: the group holding the tiles
// [acc, acc + pe) of the list (this XCD's share of it, or the whole list in the contiguous
// order) and that group's M-tile count. A workgroup locates its tiles in increasing list
// order, so the cursor only moves forward: one step per group passed, instead of a walk
// over all groups from the first for every tile (E steps of dependent scalar loads, with
// an integer division per step in the contiguous order).
struct TileCursor {
  int e;        // group
  int acc;      // list index of group e's first tile
  int pe;       // group e's tiles in the list
  int mte;      // group e's M-tiles
  int plo;      // split order: first of the group's tiles that this XCD takes
};

// RP: row groups of the columns order (see TileMap)
template <int BM, bool CONTIG, int RP>
__device__ __forceinline__ void cursor_load(TileCursor& c, const int32_t* offsets, const TileMap& m) {
  c.mte = (offsets[c.e + 1] - offsets[c.e] + BM - 1) / BM;
  if constexpr (CONTIG) {
    c.pe = c.mte * m.NT;
  } else if (m.gn > 0) {
    if constexpr (RP > 1)  // this XCD's row tiles of the group
      c.mte = row_share(c.mte, RP, (m.xcd / (kXcds / RP) + c.e) % RP);
    c.pe = c.mte * m.nx;
  } else {
    const long long pe = (long long)c.mte * m.NT;
    c.plo = (int)((pe * m.xcd) >> 3);
    c.pe = (int)((pe * (m.xcd + 1)) >> 3) - c.plo;
  }
}

template <int BM, bool CONTIG, int RP>
__device__ __forceinline__ TileCursor make_cursor(const int32_t* offsets, const TileMap& m) {
  TileCursor c;
  c.e = 0;
  c.acc = 0;
  c.plo = 0;
  cursor_load<BM, CONTIG, RP>(c, offsets, m);
  return c;
}

// Tile i of this XCD's share (see TileMap); i at or after the cursor's group, which the
// call advances. CONTIG = m.contiguous, fixed at compile time so that the split order's
// stream carries no code of the other.
template <int BM, bool CONTIG, int RP>
__device__ __forceinline__ TileCoord locate_tile(int i, const int32_t* offsets, const TileMap& m,
                                                 int bn_out, TileCursor& c) {
  const int gi = CONTIG ? m.base + i : i;
  // (the bound on the group keeps a cursor that would run past the last group in range)
  while (gi >= c.acc + c.pe && c.e < m.E - 1) {
    c.acc += c.pe;
    ++c.e;
    cursor_load<BM, CONTIG, RP>(c, offsets, m);
  }
  const int e = c.e, mte = c.mte;
  TileCoord t;
  t.e = e;
  if (!CONTIG && m.gn > 0) {
    // columns order: this XCD's rectangle of group e is mte row tiles x nx column tiles,
    // walked block by block (gn columns; only the last block may be narrower)
    const int q = gi - c.acc;
    const int g = min(q / (mte * m.gn), (m.nx - 1) / m.gn);
    const int r = q - g * mte * m.gn;
    const int wg = min(m.gn, m.nx - g * m.gn);
    const int mtl = r / wg;
    if constexpr (RP == 1) {
      t.row0 = offsets[e] + mtl * BM;
      t.rows = min(BM, offsets[e + 1] - t.row0);
      t.n0 = (m.xcd * m.nx + g * m.gn + (r - mtl * wg)) * bn_out;
    } else {
      const int rg = m.xcd / (kXcds / RP), cg = m.xcd % (kXcds / RP);
      t.row0 = offsets[e] + (mtl * RP + (rg + e) % RP) * BM;
      t.rows = min(BM, offsets[e + 1] - t.row0);
      t.n0 = (cg * m.nx + g * m.gn + (r - mtl * wg)) * bn_out;
    }
    return t;
  }
  // split: position p of the group's N-tile-major list; contiguous: the same, from the
  // group's start in the whole list
  const int p = CONTIG ? gi - c.acc : c.plo + (gi - c.acc);
  const int nt = p / mte, mtl = p - nt * mte;
  t.row0 = offsets[e] + mtl * BM;
  t.rows = min(BM, offsets[e + 1] - t.row0);
  t.n0 = nt * bn_out;
  return t;
}

// Lane id rebuilt by mbcnt inside volatile asm: per-tile copies of per-lane constants are
// recomputed from it (a few VALU ops per tile) instead of being kept live through the K
// loop, where registers are short, and reloaded from spills.
__device__ __forceinline__ int fresh_lane() {
  int ln;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
  return ln;
}

// Per-lane fragment offsets inside a stage (bytes) for substep 0. Substep s reads A
// chunk 2s + lane / 32 (swizzled), i.e. offset a_frag ^ 32 s (the chunk bits lie below
// the row bits), and B rows 16 s further down, i.e. offset b_frag + 16 s B_ROW.
template <class G, bool SWIGLU, int BNL>
__device__ __forceinline__ void frag_offsets(int ln, int wm, int wn, int (&a_frag)[G::MB],
                                             int (&b_frag)[G::NBW]) {
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb) {
    const int m = wm * G::WM + mb * 32 + (ln & 31);
    a_frag[mb] = m * (G::BK * 2) + ((ln >> 5) ^ a_swz<G::A_CPR>(m)) * 16;
  }
  const int g = ln >> 4, i = ln & 15, c = i & 3, r = i >> 2;
#pragma unroll
  for (int nb = 0; nb < G::NBW; ++nb) {
    int nbase;
    if constexpr (SWIGLU) {
      constexpr int H = G::NBW / 2;
      nbase = nb < H ? wn * (G::WNL / 2) + nb * 32 : BNL / 2 + wn * (G::WNL / 2) + (nb - H) * 32;
    } else {
      nbase = wn * G::WNL + nb * 32;
    }
    const int n = nbase + (g & 1) * 16 + 4 * c;
    const int k = (g >> 1) * 8 + r;
    const int phys = (n >> 3) ^ (b_swz(k) % G::B_SLOTS);  // the same for k + 4 and k + 16 s
    b_frag[nb] = G::A_BYTES + k * G::B_ROW + phys * 16 + ((n >> 2) & 1) * 8;
  }
}

// Gathered rows (row r of the tile is row gather[row0 + r] of A; rows past the tile's end
// repeat its last row). A wave's A loads cover 64 consecutive rows of the tile: lane l
// fetches the index of row 64 * wave + l (one load, which can be issued long before its
// use), and each load's lanes take their rows' indices from those lanes (gather_rows).
template <class G>
__device__ __forceinline__ int gather_fetch(const GemmArgs& a, const TileCoord& t, int ln, int wave) {
  // (only the gate/up GEMM gathers; other kernels compile the call on a path never taken)
  static_assert(!G::GATHERS || G::A_PW * G::A_RPI == 64, "a wave's A loads cover 64 rows");
  return a.gather[t.row0 + min(64 * wave + ln, t.rows - 1)];
}
template <class G>
__device__ __forceinline__ void gather_rows(int fetched, int ln, int (&gv)[G::A_PW]) {
#pragma unroll
  for (int j = 0; j < G::A_PW; ++j) gv[j] = __shfl(fetched, j * G::A_RPI + ln / G::A_CPR);
}

// Direct-load sources of tile t for this lane (element offsets, without the K step). With
// gathered rows, gv holds gather_rows(t).
// ks0: the first K stage the loader's stage 0 stands for (a stream-K piece starts inside K).
template <class G, bool SWIGLU, bool SPLIT, int BNL>
__device__ __forceinline__ StageLoader<G, SWIGLU, SPLIT> make_loader(const GemmArgs& a,
                                                                    const TileCoord& t, int ln,
                                                                    int wave, int nk, int ks0,
                                                                    const int (&gv)[G::A_PW]) {
  StageLoader<G, SWIGLU, SPLIT> ld;
  // gathered rows: offsets from A itself (the caller keeps every A offset below 2^31
  // elements); contiguous rows: offsets from the tile's first row
  const size_t koff = (size_t)ks0 * G::BK;
  ld.Ab = (a.gather ? a.A : a.A + (size_t)t.row0 * a.K) + koff;
  if constexpr (!SWIGLU && SPLIT) {
    // the paired tile's rows 64 .. 127 of each half are residual rows: waves 1 and 3 load
    // exactly those (64 rows per wave), from lo_rows rows further on
    static_assert(G::A_PW * G::A_RPI == 64 && G::WM == 128, "paired tile layout");
    if (wave & 1) ld.Ab += (size_t)a.lo_rows * a.K;
  }
  ld.nk = nk;
  ld.N = a.N;
  ld.wave = wave;
  const bf16* W0 = a.B0 + (size_t)t.e * a.K * a.N + koff * a.N;
  const bf16* W1 = SWIGLU ? a.B1 + (size_t)t.e * a.K * a.N + koff * a.N : W0;
#pragma unroll
  for (int j = 0; j < G::A_PW; ++j) {
    const int row = (wave * G::A_PW + j) * G::A_RPI + ln / G::A_CPR;
    const int c = (ln % G::A_CPR) ^ a_swz<G::A_CPR>(row);
    // paired down projection: tile row w * 128 + q (w = wm) holds token w * 64 + q % 64,
    // its main row for q < 64 and its residual row (wave base above) for q >= 64
    const int ar = (!SWIGLU && SPLIT) ? min((row >> 7) * 64 + (row & 63), t.rows - 1)
                   : a.gather         ? gv[j]
                                      : min(row, t.rows - 1);
    ld.a_src[j] = ar * a.K + c * 8;
  }
#pragma unroll
  for (int j = 0; j < G::B_PW; ++j) {
    const int row = (wave * G::B_PW + j) * G::B_RPI + ln / G::B_SLOTS;
    const int nl = ((ln % G::B_SLOTS) ^ (b_swz(row) % G::B_SLOTS)) * 8;
    if constexpr (SWIGLU) {
      const bool up = nl >= BNL / 2;
      ld.b_base[j] = up ? W1 : W0;
      ld.b_src[j] = row * a.N + t.n0 + (up ? nl - BNL / 2 : nl);
    } else {
      ld.b_base[j] = W0;
      ld.b_src[j] = row * a.N + t.n0 + nl;
    }
  }
  return ld;
}

template <class G>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[G::NBW][G::MB]) {
#pragma unroll
  for (int nb = 0; nb < G::NBW; ++nb)
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nb][mb][r] = 0.f;
}

// Two 8-byte pieces per lane -> one 16-byte piece: lane l < 32 keeps v[0] and takes the
// v[0] of lane l + 32; lane l + 32 takes the v[1] of lane l and keeps its own v[1].
// v_permlane32_swap exchanges the upper half-wave of its first operand with the lower
// half-wave of its second (lane layout checked on the device), so two swaps, one per
// dword, do it with no LDS traffic and no select.
__device__ __forceinline__ u32x4 swap_halves(const u32x2 (&v)[2]) {
  const auto r0 = __builtin_amdgcn_permlane32_swap(v[0][0], v[1][0], false, false);
  const auto r1 = __builtin_amdgcn_permlane32_swap(v[0][1], v[1][1], false, false);
  return u32x4{r0[0], r1[0], r0[1], r1[1]};
}

// Epilogue: acc[nb][mb][4q + i] = out[row m][col ncol + i], m = lane % 32 of block mb,
// ncol = 8q + 4 * (lane / 32) inside 32-column block nb. SwiGLU: h = silu(gate) * up in
// bf16 (and the bf16 residual of h when SPLIT); down projection: o in fp32, with SPLIT
// (paired tile) o = acc[mb] + acc[mb + MB / 2] for token wm * 64 + mb * 32 + lane % 32.
template <class G, bool SWIGLU, bool SPLIT>
__device__ __forceinline__ void store_tile(const GemmArgs& a, const TileCoord& t, int ln, int wm,
                                           int wn, const f32x16 (&acc)[G::NBW][G::MB]) {
  constexpr bool PAIRED = !SWIGLU && SPLIT;
  constexpr int MBO = PAIRED ? G::MB / 2 : G::MB;  // row blocks stored per wave
#pragma unroll
  for (int mb = 0; mb < MBO; ++mb) {
    const int m = wm * (MBO * 32) + mb * 32 + (ln & 31);
    if (m >= t.rows) continue;
    const size_t rowoff = (size_t)(t.row0 + m) * a.N + t.n0;
    if constexpr (SWIGLU) {
      constexpr int H = G::NBW / 2;
      if constexpr (!SPLIT) {
#pragma unroll
        for (int nb = 0; nb < H; ++nb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int ncol = wn * (G::WNL / 2) + nb * 32 + 8 * q + 4 * (ln >> 5);
            bf16x4 hv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float hf =
                  silu_bf16_path(acc[nb][mb][4 * q + i]) * acc[nb + H][mb][4 * q + i];
              hv[i] = (bf16)hf;
            }
            *reinterpret_cast<u32x2*>(static_cast<bf16*>(a.out) + rowoff + ncol) =
                __builtin_bit_cast(u32x2, hv);
            // one group of 4 outputs at a time: keeps the accumulator copies out of
            // AGPRs from piling up in VGPRs
            __builtin_amdgcn_sched_barrier(0);
          }
      } else {
        // h and its residual: lanes l and l + 32 swap halves so that every lane stores
        // 16 contiguous bytes of each (half the store instructions of two arrays)
#pragma unroll
        for (int nb = 0; nb < H; ++nb)
#pragma unroll
          for (int qp = 0; qp < 2; ++qp) {
            // outputs q = 2qp, 2qp + 1: lane l < 32 holds columns 16qp + 0..3 and
            // 16qp + 8..11 of its row, lane l + 32 columns 16qp + 4..7 and 16qp + 12..15;
            // one exchange leaves 16qp + 0..7 in lane l and 16qp + 8..15 in lane l + 32
            const bool hi = ln >= 32;
            u32x2 hq[2], lq[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const int q = 2 * qp + j;
              bf16x4 hv, lv;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float hf =
                    silu_bf16_path(acc[nb][mb][4 * q + i]) * acc[nb + H][mb][4 * q + i];
                hv[i] = (bf16)hf;
                lv[i] = (bf16)(hf - (float)hv[i]);
              }
              hq[j] = __builtin_bit_cast(u32x2, hv);
              lq[j] = __builtin_bit_cast(u32x2, lv);
            }
            const int ncol = wn * (G::WNL / 2) + nb * 32 + 16 * qp + (hi ? 8 : 0);
            st16(static_cast<bf16*>(a.out) + rowoff + ncol, swap_halves(hq));
            st16(static_cast<bf16*>(a.out2) + rowoff + ncol, swap_halves(lq));
            __builtin_amdgcn_sched_barrier(0);
          }
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < G::NBW; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ncol = wn * G::WNL + nb * 32 + 8 * q + 4 * (ln >> 5);
          float* const dst = static_cast<float*>(a.out) + rowoff + ncol;
          if constexpr (PAIRED) {
            f32x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = acc[nb][mb][4 * q + i] + acc[nb][mb + MBO][4 * q + i];
            *reinterpret_cast<f32x4*>(dst) = v;
          } else {
            const f32x4 v = {acc[nb][mb][4 * q + 0], acc[nb][mb][4 * q + 1],
                             acc[nb][mb][4 * q + 2], acc[nb][mb][4 * q + 3]};
            *reinterpret_cast<f32x4*>(dst) = v;
          }
        }
    }
  }
}

// ---- stream-K ----------------------------------------------------------------------
// An XCD's tile list (TileMap) is worked through by its nslot workgroups. Whole rounds of
// tiles are dealt round-robin (data-parallel: tile slot, slot + nslot, ...). The tiles of the
// last, partial round are not: their K extents, in chunks of 4 stages, are laid end to end
// and cut into nslot equal runs, one per workgroup, so that every workgroup of the XCD ends
// at the same time instead of most of them idling through a last round of few tiles. (When
// that remainder has too few chunks for the workgroups, one whole round joins it.)
//
// A run covers whole tiles and pieces of tiles. The piece that starts a tile (its "head",
// K from 0) belongs to the workgroup that owns the tile's output; the other pieces are
// computed by the following workgroups of the XCD, whose run starts inside that tile: each
// writes its fp32 accumulators to its own partial slot and raises its flag. The owner, after
// its own K loop, waits for those flags and adds the partials in workgroup order, then runs
// the epilogue. The sums therefore have one fixed order for a given shape and routing (the
// result is deterministic). A workgroup holds at most one such non-head piece (the first
// piece of its run), so one slot per workgroup suffices; a head waits only on workgroups
// after its own, so every wait ends (and a spin limit bounds it in any case). The flags are
// zero when the kernel starts (the dispatch clears them) and each owner clears the flags it
// consumed, so they are zero again when it ends.
constexpr int kSkSlots = 256;            // workgroups that may take stream-K pieces
constexpr int kSkSpinLimit = 1 << 22;    // bound on a head's wait for one partial
// Stream-K only for tiles of at least this many K stages: exchanging a piece costs a piece
// about 9 us and its owner about 35 us (256 KB partials through L2, measured per workgroup
// on the mid-size layer), which only a long tile's saved round repays. Measured (A/B in one
// process): Mixtral-size down projection (448 stages) 3197 -> 3049 us; the 128-stage
// (mid-size) and 44-stage (64-expert) down projections ran 30% and 22% slower with it.
constexpr int kSkMinStages = kStreamKMinStages;

struct SkPlan {
  int dp_tiles;   // XCD list positions [0, dp_tiles) are dealt round-robin as whole tiles
  int nkc;        // chunks (4 K stages) per tile
  int per;        // stream-K chunks per workgroup
  int c_beg, c_end;  // this workgroup's chunk run inside the stream-K part
};

__device__ __forceinline__ SkPlan make_sk_plan(int my_total, int slot, int nslot, int nk,
                                               bool enable) {
  SkPlan p;
  p.nkc = nk / 4;
  p.dp_tiles = my_total;
  p.per = 0;
  int sk_chunks = 0;
  if (enable && nk >= kSkMinStages && my_total % nslot != 0) {
    int dp = my_total / nslot * nslot;
    int rem = my_total - dp;
    if (rem * p.nkc < 2 * nslot && dp >= nslot) {  // too few chunks: add a whole round
      dp -= nslot;
      rem += nslot;
    }
    p.dp_tiles = dp;
    sk_chunks = rem * p.nkc;
    p.per = (sk_chunks + nslot - 1) / nslot;
  }
  p.c_beg = min(slot * p.per, sk_chunks);
  p.c_end = min(p.c_beg + p.per, sk_chunks);
  return p;
}

enum { kWhole = 0, kHead = 1, kPiece = 2 };
struct Item {
  int tile;      // position in the XCD's tile list
  int ks0, ks1;  // K stages [ks0, ks1)
  int role;      // kWhole, kHead (owner of a split tile), kPiece (partial for an owner)
};
struct ItemIt {
  int j;  // next round-robin round
  int c;  // next stream-K chunk
};

__device__ __forceinline__ bool next_item(ItemIt& it, const SkPlan& p, int slot, int nslot,
                                          int nk, Item& out) {
  const int i = slot + it.j * nslot;
  if (i < p.dp_tiles) {
    out.tile = i;
    out.ks0 = 0;
    out.ks1 = nk;
    out.role = kWhole;
    ++it.j;
    return true;
  }
  if (it.c < p.c_end) {
    const int u = it.c / p.nkc, kc0 = it.c - u * p.nkc;
    const int kc1 = min(p.nkc, kc0 + (p.c_end - it.c));
    out.tile = p.dp_tiles + u;
    out.ks0 = 4 * kc0;
    out.ks1 = 4 * kc1;
    out.role = kc0 > 0 ? kPiece : (kc1 < p.nkc ? kHead : kWhole);
    it.c += kc1 - kc0;
    return true;
  }
  return false;
}

// A partial slot holds one piece's fp32 accumulators as a row-major [BM, BNL] array. Only the
// down projection splits tiles: its output is the accumulator itself, so the owner, its own
// piece still in the accumulators, waits for the other pieces and stores
// o = head + p1 + p2 + ... in workgroup order, once. (The gate/up GEMM's SwiGLU epilogue would
// need the sum before it, and a second epilogue path in those kernels costs registers they do
// not have.)
//
// Where the partials travel: a piece and its owner always run on one XCD (their workgroup
// ids differ by a multiple of 8, and workgroups are dealt round-robin over a partition's 8,
// 4, 2 or 1 XCDs), so they share that XCD's L2. The partials therefore go through it: plain
// stores (the per-CU L1 writes through to L2) and loads that bypass the L1 (sc0), after the
// piece has waited for its stores to complete (vmcnt 0) and for its other waves (barrier)
// before raising the flag. The flags themselves are device-scope relaxed atomics, so a wait
// ends as soon as the flag is raised whatever the placement. (Device-scope accesses for the
// partials, sc1, write through to memory and ran at about 10 GB/s per CU; a device-scope
// release or acquire fence writes back or invalidates the whole L2 of the XCD.)
constexpr int kCpolSc0 = 1;                  // cache-policy bits: miss in the per-CU L1
constexpr int kBufRsrcWord3 = 0x00020000;    // raw buffer descriptor, dword 3

__device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rsrc(const GemmArgs& a, int slot_id) {
  return __builtin_amdgcn_make_buffer_rsrc(a.partial + (size_t)slot_id * (kStreamKSlotBytes / 4),
                                           0, (int)kStreamKSlotBytes, kBufRsrcWord3);
}

template <class G>
__device__ __forceinline__ void put_partial(const GemmArgs& a, int bid, int ln, int wm, int wn,
                                            const f32x16 (&acc)[G::NBW][G::MB]) {
  constexpr int BNL = G::WNL * G::WGN;
  const __amdgpu_buffer_rsrc_t r = partial_rsrc(a, bid);
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb) {
    const int m = wm * G::WM + mb * 32 + (ln & 31);
#pragma unroll
    for (int nb = 0; nb < G::NBW; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ncol = wn * G::WNL + nb * 32 + 8 * q + 4 * (ln >> 5);
        const f32x4 v = {acc[nb][mb][4 * q + 0], acc[nb][mb][4 * q + 1], acc[nb][mb][4 * q + 2],
                         acc[nb][mb][4 * q + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(v, r, (m * BNL + ncol) * 4, 0, 0);
      }
  }
  wait_vmcnt<0>();   // this thread's partial stores have reached the L2
  __syncthreads();   // and every other thread's
  if (threadIdx.x == 0)
    __hip_atomic_store(a.flags + bid, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The owner of a split tile, with its own piece still in the accumulators: wait for the
// pieces of the later workgroups of this XCD whose runs cover the rest of the tile
// (w = slot + 1 .. w_last; thread 0 waits for each flag and clears it), then store
// o = head + p_{slot+1} + p_{slot+2} + ... element by element, in that order: one store of
// o and one read of each partial. (Storing the head first and adding the partials to o after
// it wrote o twice and read it back, 1 MB per tile split in two against 512 KB here; the same
// additions in the same order, so the same bits.)
template <class G>
__device__ __forceinline__ void store_tile_sum(const GemmArgs& a, const TileCoord& t, int xcd,
                                               int slot, int w_last, int ln, int wm, int wn,
                                               const f32x16 (&acc)[G::NBW][G::MB]) {
  constexpr int BNL = G::WNL * G::WGN;
  if (threadIdx.x == 0) {
    for (int w = slot + 1; w <= w_last; ++w) {
      const int wb = w * kXcds + xcd;
      int n = 0;
      while (__hip_atomic_load(a.flags + wb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0 &&
             ++n < kSkSpinLimit)
        __builtin_amdgcn_s_sleep(8);
      __hip_atomic_store(a.flags + wb, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  float* o = static_cast<float*>(a.out);
  // per 32-row block and quarter of its columns: 8 chunks of each partial are loaded before
  // they are added (a running sum and one partial in flight: 64 VGPRs)
  constexpr int NQ = G::NBW * 4, NH = 4, HQ = NQ / NH;
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb) {
    const int m = wm * G::WM + mb * 32 + (ln & 31);
    const bool row_ok = m < t.rows;
    const size_t rowoff = (size_t)(t.row0 + (row_ok ? m : 0)) * a.N + t.n0;
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      f32x4 v[HQ];
#pragma unroll
      for (int ii = 0; ii < HQ; ++ii) {
        const int i = hh * HQ + ii, nb = i / 4, q = i % 4;
        v[ii] = f32x4{acc[nb][mb][4 * q + 0], acc[nb][mb][4 * q + 1], acc[nb][mb][4 * q + 2],
                      acc[nb][mb][4 * q + 3]};
      }
      for (int w = slot + 1; w <= w_last; ++w) {
        const __amdgpu_buffer_rsrc_t r = partial_rsrc(a, w * kXcds + xcd);
        f32x4 p[HQ];
#pragma unroll
        for (int ii = 0; ii < HQ; ++ii) {
          const int i = hh * HQ + ii;
          const int ncol = wn * G::WNL + (i / 4) * 32 + 8 * (i % 4) + 4 * (ln >> 5);
          p[ii] = __builtin_amdgcn_raw_buffer_load_b128(r, (m * BNL + ncol) * 4, 0, kCpolSc0);
        }
#pragma unroll
        for (int ii = 0; ii < HQ; ++ii) v[ii] += p[ii];
      }
      if (row_ok) {
#pragma unroll
        for (int ii = 0; ii < HQ; ++ii) {
          const int i = hh * HQ + ii;
          const int ncol = wn * G::WNL + (i / 4) * 32 + 8 * (i % 4) + 4 * (ln >> 5);
          *reinterpret_cast<f32x4*>(o + rowoff + ncol) = v[ii];
        }
      }
      // one batch at a time: keeps the accumulator copies from piling up in VGPRs
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// This workgroup's work items (whole tiles, then its stream-K run) as one stream of K stages
// through the ring (PipeStep): the last S steps of an item refill the ring with the next
// item's first S stages, so those loads are in flight while this item's epilogue runs and
// the next item only waits for its stage 0 to be read. Every item's stage count is a
// multiple of S (whole chunks), so that stage s of every item sits in ring buffer s % S.
// (The next item's fragments are read after the epilogue: holding them through it would
// leave too few registers.)
// (TR: rows of the grouped problem per tile; TAG: see k_loop)
template <class G, bool SWIGLU, bool SPLIT, int TR, int BNL, bool CONTIG, int RP, int TAG>
__device__ __forceinline__ void pipe_stream(const GemmArgs& a, const TileMap& tm, int slot,
                                            int nslot, int wave, int wm, int wn, int nk,
                                            char* const (&ring)[G::STAGES]) {
  constexpr int S = G::STAGES;
  static_assert(S == 4, "the pipelined loop is written out for a ring of 4");
  // stream-K: the plain down projection only (paired tiles sum in the epilogue)
  constexpr bool SK = !SWIGLU && !SPLIT;
  const SkPlan sp = make_sk_plan(tm.my_total, slot, nslot, nk, SK && a.partial != nullptr);
  ItemIt it{0, sp.c_beg};
  Item cur;
  if (!next_item(it, sp, slot, nslot, nk, cur)) return;
  int ln = fresh_lane();
  int a_frag[G::MB], b_frag[G::NBW];
  frag_offsets<G, SWIGLU, BNL>(ln, wm, wn, a_frag, b_frag);
  TileCursor cur_c = make_cursor<TR, CONTIG, RP>(a.offsets, tm);
  TileCoord t = locate_tile<TR, CONTIG, RP>(cur.tile, a.offsets, tm, G::BN_OUT, cur_c);
  int gv[G::A_PW] = {};
  if (SWIGLU && a.gather) gather_rows<G>(gather_fetch<G>(a, t, ln, wave), ln, gv);
  StageLoader<G, SWIGLU, SPLIT> ld =
      make_loader<G, SWIGLU, SPLIT, BNL>(a, t, ln, wave, nk, cur.ks0, gv);
#define MOE_SSTEP(J, RL, RSTAGE)                                                             \
  PipeStep<G, SWIGLU, SPLIT, J, true>::run(0, true, true, RL, RSTAGE, ring, a_frag, b_frag, acc, \
                                       (J) % 2 ? F1 : F0, (J) % 2 ? F0 : F1)
  // prologue of the first item: the whole ring in flight
#pragma unroll
  for (int i = 0; i < S; ++i) ld.issue(i, ring[i]);
  for (;;) {
    // accumulators and fragments are per item (none is carried around this loop)
    f32x16 acc[G::NBW][G::MB];
    zero_acc<G>(acc);
    Frags<G> F0, F1;
    // stage 0's fragments (the ring holds stages 0 .. S-1 of this item, stage 0 is the
    // oldest load in flight; epilogue stores of the previous item may be newer)
    wait_vmcnt<(S - 1) * G::LPS>();
    sync_point();
#pragma unroll
    for (int r = 0; r < G::SUB * G::MB + 2 * G::SUB * G::NBW; ++r)
      read_frag<G>(r, ring[0], a_frag, b_frag, F0);
    // the next item (this one again after the last: its loads below are unused but in
    // bounds)
    Item nx = cur;
    const bool has_next = next_item(it, sp, slot, nslot, nk, nx);
    const TileCoord tn =
        has_next ? locate_tile<TR, CONTIG, RP>(nx.tile, a.offsets, tm, G::BN_OUT, cur_c) : t;
    // gathered rows: the next tile's row indices, fetched now so that the load is long
    // complete when they are needed (a vector load completes in order with the ring's
    // loads; one issued just before its use would wait for all of them)
    const int gnext = (SWIGLU && a.gather) ? gather_fetch<G>(a, tn, fresh_lane(), wave) : 0;
    const int nkt = cur.ks1 - cur.ks0;
    int kt = 0;
    for (; kt + 2 * S <= nkt; kt += S) {  // refills from this item
      MOE_SSTEP(0, ld, kt + S);
      MOE_SSTEP(1, ld, kt + S + 1);
      MOE_SSTEP(2, ld, kt + S + 2);
      MOE_SSTEP(3, ld, kt + S + 3);
    }
    // kt == nkt - S: the last S steps refill the ring with the next item's first S
    // stages; after the last item they load this item's first stages again, unused but
    // in bounds, so that every path into the loop above has the same loads in flight
    // (the compiler then needs no extra wait there). The last step reads nothing.
    ln = fresh_lane();
    if (SWIGLU && a.gather) gather_rows<G>(gnext, ln, gv);
    const StageLoader<G, SWIGLU, SPLIT> ldn =
        make_loader<G, SWIGLU, SPLIT, BNL>(a, tn, ln, wave, nk, nx.ks0, gv);
    MOE_SSTEP(0, ldn, 0);
    MOE_SSTEP(1, ldn, 1);
    MOE_SSTEP(2, ldn, 2);
    PipeStep<G, SWIGLU, SPLIT, 3, false>::run(S - 2, false, true, ldn, 3, ring, a_frag, b_frag,
                                              acc, F1, F0);
    ln = fresh_lane();
    if (SK && cur.role == kPiece) {
      put_partial<G>(a, (int)blockIdx.x, ln, wm, wn, acc);
    } else if (SK && cur.role == kHead) {
      // the workgroups whose runs cover the rest of this tile
      const int u = cur.tile - sp.dp_tiles;
      store_tile_sum<G>(a, t, (int)blockIdx.x & (kXcds - 1), slot,
                        ((u + 1) * sp.nkc - 1) / sp.per, ln, wm, wn, acc);
    } else {
      store_tile<G, SWIGLU, SPLIT>(a, t, ln, wm, wn, acc);
    }
    if (!has_next) break;
    t = tn;
    ld = ldn;
    cur = nx;
  }
#undef MOE_SSTEP
  wait_vmcnt<0>();
}

template <int BM, int BNL, bool SWIGLU, bool SPLIT, int NW, bool CONTIG_OK, int RP>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void gemm_bf16_kernel(
    const bf16* __restrict__ A, const int32_t* __restrict__ gather, const bf16* __restrict__ B0,
    const bf16* __restrict__ B1, const int32_t* __restrict__ offsets, int E, int K, int N, int lo_rows,
    void* __restrict__ out, void* __restrict__ out2, int gn, float* __restrict__ partial,
    int32_t* __restrict__ flags) {
  using G = Geo<BM, BNL, SWIGLU, SPLIT, NW>;
  // one array per ring stage, so that the compiler can tell a stage's LDS reads from
  // the direct loads still in flight into the other stages
  __shared__ __attribute__((aligned(1024))) char lds0[G::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char lds1[G::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char lds2[G::STAGES > 2 ? G::STAGE_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char lds3[G::STAGES > 3 ? G::STAGE_BYTES : 16];
  char* const ring4[4] = {lds0, lds1, lds2, lds3};
  char* ring[G::STAGES];
#pragma unroll
  for (int i = 0; i < G::STAGES; ++i) ring[i] = ring4[i];
  // the wave index is uniform: keep it scalar so LDS destinations stay plain offsets
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int wm = wave / G::WGN, wn = wave % G::WGN;
  // one wave per SIMD on 256 (or 192) x 256 tiles: the software-pipelined loop
  constexpr bool PIPE = NW == 4 && (BM == 256 || BM == 192) && BNL == 256;
  // rows of the grouped problem per tile: BM, or BM / 2 tokens in the paired down projection
  constexpr bool PAIRED = !SWIGLU && SPLIT;
  constexpr int TR = PAIRED ? BM / 2 : BM;

  const int NT = N / G::BN_OUT;
  const int xcd = blockIdx.x & (kXcds - 1), slot = blockIdx.x / kXcds, nslot = gridDim.x / kXcds;
  // this XCD's tiles (the order is described at TileMap)
  const TileMap tm = make_tile_map<TR, CONTIG_OK, RP>(offsets, E, NT, xcd, gather != nullptr, gn);
  // (one instantiation of the shared helpers per kernel: see k_loop)
  constexpr int TAG = (CONTIG_OK ? 1 : 0) + 2 * (RP - 1);
  const int my_total = tm.my_total;
  const int nk = K / G::BK;
  const int nk_total = nk;

  // (no stream-K in the paired down projection: a piece's partial sums would need the pair
  // sum of the epilogue)
  const GemmArgs args{A, gather, B0, B1, offsets, E, K, N, out, out2,
                      PIPE && BM == 256 && !PAIRED && gridDim.x <= kSkSlots ? partial : nullptr,
                      flags,
                      lo_rows};
  if constexpr (PIPE) {
    if (nk_total % G::STAGES == 0 && nk_total >= 2 * G::STAGES) {
      if (CONTIG_OK && tm.contiguous)
        pipe_stream<G, SWIGLU, SPLIT, TR, BNL, CONTIG_OK, RP, TAG>(args, tm, slot, nslot, wave,
                                                                   wm, wn, nk, ring);
      else
        pipe_stream<G, SWIGLU, SPLIT, TR, BNL, false, RP, TAG>(args, tm, slot, nslot, wave, wm,
                                                               wn, nk, ring);
      return;
    }
  }
  TileCursor cur_c = make_cursor<TR, false, RP>(offsets, tm);
  TileCursor cur_cc = make_cursor<TR, CONTIG_OK, RP>(offsets, tm);
  for (int i = slot; i < my_total; i += nslot) {
    const int ln = fresh_lane();
    int a_frag[G::MB], b_frag[G::NBW];
    frag_offsets<G, SWIGLU, BNL>(ln, wm, wn, a_frag, b_frag);
    const TileCoord t = CONTIG_OK && tm.contiguous
                            ? locate_tile<TR, CONTIG_OK, RP>(i, offsets, tm, G::BN_OUT, cur_cc)
                            : locate_tile<TR, false, RP>(i, offsets, tm, G::BN_OUT, cur_c);
    int gv[G::A_PW] = {};
    if (SWIGLU && args.gather) gather_rows<G>(gather_fetch<G>(args, t, ln, wave), ln, gv);
    const StageLoader<G, SWIGLU, SPLIT> ld = make_loader<G, SWIGLU, SPLIT, BNL>(args, t, ln, wave, nk, 0, gv);
    f32x16 acc[G::NBW][G::MB];
    zero_acc<G>(acc);

    // (the pipelined layout falls back to the plain ring when its stream does not apply)
    k_loop<G, SWIGLU, SPLIT, TAG>(nk_total, ring, ld, a_frag, b_frag, acc);

    store_tile<G, SWIGLU, SPLIT>(args, t, ln, wm, wn, acc);
    // stores retired and every wave past its last stage read before the next tile's
    // loads refill the ring
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
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

// Column-block width of the columns tile order (0: split order). An XCD's 32 concurrent tiles
// span about 32 / GN row tiles and GN column tiles, so about 32 / GN + GN tile operands are
// fetched per 32 tiles. Measured on the Mixtral-size layer (NX = 14 gate/up columns per XCD,
// A/B in one process): widths 3 to 7 within 1% of each other, 4 the best, all 4-5% faster
// than the split order; NX = 2 (its down projection): width 2 is 2% faster than 1 or split.
// NX columns are cut into round(NX / 4) blocks.
int column_block(int NT, int rp) {
  if (NT % kXcds != 0) return 0;
  const int nx = NT * rp / kXcds;
  const int nblocks = nx < 6 ? 1 : (nx + 2) / 4;
  return (nx + nblocks - 1) / nblocks;
}

// Row groups of the columns order (1 or 2). Every row tile is fetched by the 8 / RP XCDs of its
// row group and every weight column by RP XCDs, so about RP * W + (8 / RP) * A elements move
// beyond L2 (A: the rows, rows x K; W: the weights, E x K x N); two row groups fetch less when
// W < 4 A. Measured on a one-expert down projection of 4096 rows, K = 14336, N = 4096 (rows
// and weights alike): one row group fetched 9 times the rows' bytes, which the model gives.
int row_groups(int NT, long long rows, int K, int N, int E) {
  if (NT % kXcds != 0) return 1;
  const double A = (double)rows * K, W = (double)E * K * N;
  return W < 4.0 * A ? 2 : 1;
}

// rows: the grouped problem's rows (at most), for the choice of row groups
template <int BM, int BNL, bool SWIGLU, bool SPLIT, int NW>
hipError_t launch_bf16(const void* A, const int32_t* gather, const void* B0, const void* B1,
                       const int32_t* offsets, int E, long long rows, int K, int N, void* out,
                       void* out2, int lo_rows, const StreamK& sk, hipStream_t s) {
  const int grid = ((device_cu_count() + 7) / 8) * 8;
  // a non-empty group has at least N / BN_OUT tiles: the contiguous order is possible
  // only below the threshold (kernels for wider outputs are built without it; split-order
  // shapes between kContigTiles and kContigSplitTiles column tiles forgo it)
  const int NT = N / (SWIGLU ? BNL / 2 : BNL);
  // (two row groups only for plain-row down projections too wide for the contiguous order:
  // the only kernels built with them)
  const int rp = !SWIGLU && !SPLIT && NT >= kContigTiles ? row_groups(NT, rows, K, N, E) : 1;
  const int gn = column_block(NT, rp);
#define MOE_GEMM_BF16(CONTIG, RPV)                                                              \
  gemm_bf16_kernel<BM, BNL, SWIGLU, SPLIT, NW, CONTIG, RPV><<<grid, 64 * NW, 0, s>>>(             \
      static_cast<const bf16*>(A), gather, static_cast<const bf16*>(B0),                          \
      static_cast<const bf16*>(B1), offsets, E, K, N, lo_rows, out, out2, gn, sk.partial, sk.flags)
  if (NT < (gather ? kContigGatherTiles : kContigTiles)) {
    MOE_GEMM_BF16(true, 1);
  } else if constexpr (!SWIGLU && !SPLIT) {
    if (rp == 2) MOE_GEMM_BF16(false, 2);
    else MOE_GEMM_BF16(false, 1);
  } else {
    MOE_GEMM_BF16(false, 1);
  }
#undef MOE_GEMM_BF16
  return hipGetLastError();
}

template <bool SPLIT>
hipError_t gateup_bf16(const void* xp, const int32_t* gather, const void* Wgate, const void* Wup,
                       const int32_t* offsets, int E, int R_max, int d, int f, void* h,
                       void* h_lo, const StreamK& sk, hipStream_t s) {
  if (f % 128 == 0)
    return launch_bf16<256, 256, true, SPLIT, 4>(xp, gather, Wgate, Wup, offsets, E, R_max, d, f, h,
                                                 h_lo, 0, sk, s);
  return launch_bf16<256, 128, true, SPLIT, 4>(xp, gather, Wgate, Wup, offsets, E, R_max, d, f, h,
                                               h_lo, 0, sk, s);
}

// Whether the down projection of up to R_max rows in E groups fits one round of the
// workgroups in 192-row tiles (at most R_max / 192 + E row tiles). A layer whose 256-row
// tiles already fit one round, or nearly, then finishes when its slowest tile does, and a
// 192-row tile is three quarters of the work: the mid-size layer (8192 rows, 8 experts,
// d_model 1024) runs 140 tiles of 256 rows on 256 CUs, or about 190 of 192.
bool down_fits_192(long long R_max, int E, int d) {
  const long long tiles = (R_max / 192 + E) * (long long)(d / 256);
  return tiles <= ((device_cu_count() + 7) / 8) * 8;
}

// PAIRED: h's residual rows sit lo_rows rows after their main rows (see store_tile)
template <bool PAIRED>
hipError_t down_bf16(const void* h, const void* Wdown, const int32_t* offsets, int E, int R_max,
                     int f, int d, float* o, int lo_rows, const StreamK& sk, hipStream_t s) {
  // (the paired tiles read each row and its residual row)
  const long long rows = PAIRED ? 2LL * R_max : R_max;
  if (!PAIRED && d % 256 == 0 && down_fits_192(R_max, E, d))
    return launch_bf16<192, 256, false, false, 4>(h, nullptr, Wdown, nullptr, offsets, E, rows, f, d,
                                                  o, nullptr, 0, sk, s);
  if (d % 256 == 0)
    return launch_bf16<256, 256, false, PAIRED, 4>(h, nullptr, Wdown, nullptr, offsets, E, rows, f, d,
                                                   o, nullptr, lo_rows, sk, s);
  if (d % 128 == 0)
    return launch_bf16<256, 128, false, PAIRED, 4>(h, nullptr, Wdown, nullptr, offsets, E, rows, f, d,
                                                   o, nullptr, lo_rows, sk, s);
  return launch_bf16<256, 64, false, PAIRED, 4>(h, nullptr, Wdown, nullptr, offsets, E, rows, f, d, o,
                                                nullptr, lo_rows, sk, s);
}

}  // namespace

hipError_t launch_gemm_gateup(int bf16in, const void* xp, const int32_t* gather, const void* Wgate,
                              const void* Wup, const int32_t* offsets, int E, int R_max, int d,
                              int f, void* h, void* h_lo, const StreamK& sk, hipStream_t s) {
  if (bf16in) {
    if (h_lo)
      return gateup_bf16<true>(xp, gather, Wgate, Wup, offsets, E, R_max, d, f, h, h_lo, sk, s);
    return gateup_bf16<false>(xp, gather, Wgate, Wup, offsets, E, R_max, d, f, h, nullptr, sk, s);
  }
  if (gather) return hipErrorInvalidValue;  // the fp32 path reads copied rows
  dim3 grid(f / 64, R_max / 64 + E);
  gemm_f32_kernel<true><<<grid, 256, 0, s>>>(static_cast<const float*>(xp),
                                             static_cast<const float*>(Wgate),
                                             static_cast<const float*>(Wup), offsets, E, d, f,
                                             static_cast<float*>(h));
  return hipGetLastError();
}

hipError_t launch_gemm_down(int bf16in, const void* h, const void* Wdown, const int32_t* offsets,
                            int E, int R_max, int f, int d, float* o, int lo_rows,
                            const StreamK& sk, hipStream_t s) {
  if (bf16in) {
    if (lo_rows > 0) return down_bf16<true>(h, Wdown, offsets, E, R_max, f, d, o, lo_rows, sk, s);
    return down_bf16<false>(h, Wdown, offsets, E, R_max, f, d, o, 0, sk, s);
  }
  if (lo_rows > 0) return hipErrorInvalidValue;  // the fp32 path has no residual rows
  dim3 grid(d / 64, R_max / 64 + E);
  gemm_f32_kernel<false><<<grid, 256, 0, s>>>(static_cast<const float*>(h),
                                              static_cast<const float*>(Wdown), nullptr, offsets,
                                              E, f, d, o);
  return hipGetLastError();
}
