// Host side of the C ABI (include/moe.h): argument checks, workspace layout and the
// launch sequence on the caller's stream. No allocation, no synchronisation.
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "api_internal.h"
#include "kernels.h"
#include "moe.h"

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

struct Layout {
  int64_t R = 0, C = 0;
  int nblk = 0;
  size_t idx = 0, w = 0, lrank = 0, pos = 0, src = 0, blk_counts = 0, blk_psum = 0, base = 0,
         offsets = 0, counts = 0, logitsT = 0, blk_zsum = 0, x_perm = 0, h = 0, h_lo = 0, o = 0,
         sk_partial = 0, sk_flags = 0, ec_runs = 0, total = 0;
  bool stream_k = false;  // bf16: the GEMMs' stream-K partial slots and flags exist
  bool xperm = false;  // rows copied into x_perm (else the gate/up GEMM gathers them from x)
};

int64_t ec_capacity(const moe_shape& s) {
  const double c = floor((double)s.T * s.capacity_factor / (double)s.E);
  if (!(c >= 0.0) || c > 9.0e18) return -1;
  return (int64_t)c;
}

// Token choice with an expert capacity: int((T / E) * cf * k), the product taken in that
// order in double (机器学习基础系列——混合专家模型, expert_capacity_routing).
int64_t tc_capacity(const moe_shape& s) {
  const double c = floor((double)s.T / (double)s.E * s.capacity_factor * (double)s.k);
  if (!(c >= 0.0) || c > 9.0e18) return -1;
  return (int64_t)c;
}

bool is_tc(int32_t mode) { return mode == MOE_TOKEN_CHOICE || mode == MOE_TOKEN_CHOICE_CAPACITY; }

// Per-expert slot limit handed to the dispatch: INT_MAX without a capacity.
int tc_cap_limit(const moe_shape& s) {
  if (s.mode != MOE_TOKEN_CHOICE_CAPACITY) return INT_MAX;
  const int64_t c = tc_capacity(s);
  return c >= (int64_t)INT_MAX ? INT_MAX - 1 : (int)c;
}

moe_status check_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_NULL_ARG;
  if (s->dtype != MOE_FP32 && s->dtype != MOE_BF16) return MOE_ERR_BAD_SHAPE;
  if (s->mode != MOE_TOKEN_CHOICE && s->mode != MOE_EXPERT_CHOICE &&
      s->mode != MOE_TOKEN_CHOICE_CAPACITY)
    return MOE_ERR_BAD_SHAPE;
  if (s->T < 0 || s->d_model <= 0 || s->d_ff <= 0 || s->E < 1) return MOE_ERR_BAD_SHAPE;
  // every row index is an int32 (and T * k below must not overflow)
  if (s->T >= (int64_t(1) << 31)) return MOE_ERR_BAD_SHAPE;
  if (s->d_model > (1 << 20) || s->d_ff > (1 << 20)) return MOE_ERR_BAD_SHAPE;
  // a limit of the kernels' tiles (whole 64-column tiles, whole 32-deep K stages), not of
  // the method
  if (s->d_model % 64 || s->d_ff % 64) return MOE_ERR_UNSUPPORTED;
  if (s->E > 64) return MOE_ERR_UNSUPPORTED;
  if (is_tc(s->mode)) {
    if (s->k < 1 || s->k > s->E) return MOE_ERR_BAD_SHAPE;
    if (s->k > 8) return MOE_ERR_UNSUPPORTED;
    if (s->renormalize != 0 && s->renormalize != 1) return MOE_ERR_BAD_SHAPE;
    if (s->T * (int64_t)s->k >= (int64_t(1) << 31)) return MOE_ERR_BAD_SHAPE;
    if (s->mode == MOE_TOKEN_CHOICE_CAPACITY) {
      if (!(s->capacity_factor > 0.0) || !isfinite(s->capacity_factor)) return MOE_ERR_BAD_SHAPE;
      if (tc_capacity(*s) < 0) return MOE_ERR_BAD_SHAPE;
    }
  } else {
    if (!(s->capacity_factor > 0.0) || !isfinite(s->capacity_factor)) return MOE_ERR_BAD_SHAPE;
    const int64_t C = ec_capacity(*s);
    if (C < 1 || C > s->T) return MOE_ERR_BAD_SHAPE;
    if (C * (int64_t)s->E >= (int64_t(1) << 31)) return MOE_ERR_BAD_SHAPE;
  }
  // the fp32 GEMMs launch one grid row per 64 routed rows (plus one per group): the grid's
  // y extent bounds the rows they take
  if (s->dtype == MOE_FP32) {
    const int64_t rows = is_tc(s->mode) ? s->T * (int64_t)s->k : ec_capacity(*s) * s->E;
    if (rows / 64 + s->E > 65535) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

Layout make_layout(const moe_shape& s) {
  Layout L;
  const size_t eb = s.dtype == MOE_BF16 ? 2 : 4;
  const int64_t T = s.T, E = s.E, d = s.d_model, f = s.d_ff;
  size_t cur = 0;
  auto take = [&](size_t bytes) {
    const size_t at = cur;
    cur = align_up(cur + bytes);
    return at;
  };
  L.nblk = (int)((T + 63) / 64);
  if (is_tc(s.mode)) {
    const int64_t k = s.k;
    L.R = T * k;
    L.idx = take(T * k * 4);
    L.w = take(T * k * 4);
    L.lrank = take(T * k * 4);
    L.pos = take(T * k * 4);
    L.blk_counts = take((size_t)L.nblk * E * 4);
    L.blk_psum = take((size_t)L.nblk * E * 4);
    L.base = take((size_t)L.nblk * E * 4);
  } else {
    L.C = ec_capacity(s);
    L.R = E * L.C;
    L.logitsT = take(E * T * 4);
    L.idx = take(L.R * 4);
    L.w = take(L.R * 4);
  }
  L.blk_zsum = take((size_t)L.nblk * 4);
  // expert choice, bf16: h's bf16 rounding residual is carried as rows R .. 2R-1 of the
  // h region; the down projection takes each row with its residual row and writes their
  // products' sum
  const bool resid = s.mode == MOE_EXPERT_CHOICE && s.dtype == MOE_BF16;
  const int64_t hrows = resid ? 2 * L.R : L.R;
  L.offsets = take((size_t)(E + 1) * 4);
  L.counts = take(E * 4);
  L.src = take(L.R * 4);
  // bf16: the gate/up GEMM loads its rows straight from x through src (per-lane addresses of
  // its direct-to-LDS loads) while every row offset fits in 31 bits; otherwise (and in
  // fp32) the permute copies the rows into x_perm
  L.xperm = !(s.dtype == MOE_BF16 && T * d < (int64_t(1) << 31));
  if (L.xperm) L.x_perm = take((size_t)L.R * d * eb);
  L.h = take((size_t)hrows * f * eb);
  if (resid) L.h_lo = L.h + (size_t)L.R * f * eb;
  L.o = take((size_t)L.R * d * 4);
  // the bf16 down projection splits the tiles of its last partial round along K (stream-K)
  // when they have kStreamKMinStages K stages or more: one fp32 partial slot and one flag
  // per workgroup (not with the residual rows, whose pairs are summed in the epilogue)
  L.stream_k = s.dtype == MOE_BF16 && !resid && f / 32 >= kStreamKMinStages;
  if (L.stream_k) {
    L.sk_partial = take((size_t)kStreamKSlots * kStreamKSlotBytes);
    L.sk_flags = take((size_t)kStreamKSlots * 4);
  }
  // expert choice: the select's run table for the combine (entries of each expert's list
  // before each block of kEcCombineTokens tokens); last, so that the buffers above keep the
  // offsets they have without it
  if (!is_tc(s.mode)) L.ec_runs = take((size_t)E * ec_run_stride((int)T) * 4);
  L.total = cur;
  return L;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Training noise: token choice only; the draw given (eps) or drawn in the router kernel
// (eps null: seed, offset, a finite scale), W_noise optional.
moe_status check_noise(const moe_shape& s, const moe_noise* noise) {
  if (!noise) return MOE_OK;
  if (!is_tc(s.mode)) return MOE_ERR_UNSUPPORTED;
  if (!noise->eps && !isfinite(noise->scale)) return MOE_ERR_BAD_SHAPE;
  if (!aligned16(noise->W_noise) || !aligned16(noise->eps)) return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

// ---- stage timing ----------------------------------------------------------------
struct ProfRec {
  int stage;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof_recs;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t prof_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

struct StageTimer {
  int stage;
  hipStream_t s;
  hipEvent_t a = nullptr, b = nullptr;
  StageTimer(int st, hipStream_t str) : stage(st), s(str) {
    std::lock_guard<std::mutex> g(g_prof_mu);
    if (!g_prof_on) return;
    a = prof_event();
    b = prof_event();
    if (!a || !b || hipEventRecord(a, s) != hipSuccess) drop();
  }
  void drop() {
    if (a) g_event_pool.push_back(a);
    if (b) g_event_pool.push_back(b);
    a = b = nullptr;
  }
  void done() {
    if (!a || !b) return;
    const bool ok = hipEventRecord(b, s) == hipSuccess;
    std::lock_guard<std::mutex> g(g_prof_mu);
    if (ok) g_prof_recs.push_back({stage, a, b});
    else drop();
    a = b = nullptr;
  }
};

#define MOE_LAUNCH(stage, call)              \
  do {                                       \
    StageTimer _t((stage), stream);          \
    hipError_t _e = (call);                  \
    _t.done();                               \
    if (_e != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

moe_status zero_stats(int E, float* f, float* p, float* loss, int32_t* counts, float* z_loss,
                      hipStream_t stream) {
  if (z_loss) MOE_LAUNCH(MOE_STAGE_AUX, launch_fill_zero(z_loss, 4, stream));
  if (f) MOE_LAUNCH(MOE_STAGE_AUX, launch_fill_zero(f, (size_t)E * 4, stream));
  if (p) MOE_LAUNCH(MOE_STAGE_AUX, launch_fill_zero(p, (size_t)E * 4, stream));
  if (loss) MOE_LAUNCH(MOE_STAGE_AUX, launch_fill_zero(loss, 4, stream));
  if (counts) MOE_LAUNCH(MOE_STAGE_AUX, launch_fill_zero(counts, (size_t)E * 4, stream));
  return MOE_OK;
}

// Token-choice dispatch after the router: group offsets, counts, the requested statistics
// (f, p, loss, z_loss), the slots' rows (pos, src), capacity drops and renormalised weights,
// row copies into x_perm (when not nullptr) and the stream-K flags cleared (when not
// nullptr). Up to kFusedMaxBlocks router blocks in one kernel; beyond, the dispatch scan and
// then (when `permute` is set) the permute kernel.
moe_status run_dispatch_tc(const moe_shape& s, const Layout& L, const void* x, int32_t* idx,
                           float* w, int32_t* user_counts, float* f, float* p, float* loss,
                           float* z_loss, void* x_perm, int32_t* sk_flags, bool permute, void* ws,
                           hipStream_t stream) {
  const bool want_z = z_loss != nullptr;
  const int eb = s.dtype == MOE_BF16 ? 2 : 4;
  if (L.nblk <= kFusedMaxBlocks) {
    DispatchArgs da{};
    da.x = static_cast<const char*>(x);
    da.elt_bytes = eb;
    da.T = (int)s.T;
    da.d = (int)s.d_model;
    da.E = s.E;
    da.k = s.k;
    da.nblk = L.nblk;
    da.cap = tc_cap_limit(s);
    da.renorm = s.renormalize;
    da.idx = idx;
    da.lrank = at<int32_t>(ws, L.lrank);
    da.blk_counts = at<int32_t>(ws, L.blk_counts);
    da.pos = at<int32_t>(ws, L.pos);
    da.src = at<int32_t>(ws, L.src);
    da.w = w;
    da.x_perm = static_cast<char*>(x_perm);
    da.offsets = at<int32_t>(ws, L.offsets);
    da.counts = at<int32_t>(ws, L.counts);
    da.user_counts = user_counts;
    da.blk_psum = at<float>(ws, L.blk_psum);
    da.blk_zsum = want_z ? at<float>(ws, L.blk_zsum) : nullptr;
    da.f = f;
    da.p = p;
    da.loss = loss;
    da.z_loss = z_loss;
    da.sk_flags = sk_flags;
    MOE_LAUNCH(MOE_STAGE_PERMUTE, launch_dispatch_tc(da, stream));
    return MOE_OK;
  }
  ScanArgs sa{};
  sa.blk_counts = at<int32_t>(ws, L.blk_counts);
  sa.nblk = L.nblk;
  sa.E = s.E;
  sa.cap = tc_cap_limit(s);
  sa.counts = at<int32_t>(ws, L.counts);
  sa.offsets = at<int32_t>(ws, L.offsets);
  sa.base = at<int32_t>(ws, L.base);
  sa.user_counts = user_counts;
  sa.blk_psum = at<float>(ws, L.blk_psum);
  sa.blk_zsum = want_z ? at<float>(ws, L.blk_zsum) : nullptr;
  sa.T = (int)s.T;
  sa.k = s.k;
  sa.f = f;
  sa.p = p;
  sa.loss = loss;
  sa.z_loss = z_loss;
  MOE_LAUNCH(MOE_STAGE_SCAN, launch_dispatch_scan(sa, stream));
  if (!permute) return MOE_OK;
  MOE_LAUNCH(MOE_STAGE_PERMUTE,
             launch_permute_tc(x, eb, (int)s.T, (int)s.d_model, s.E, s.k, idx,
                               at<int32_t>(ws, L.lrank), at<int32_t>(ws, L.base),
                               at<int32_t>(ws, L.offsets), tc_cap_limit(s), s.renormalize,
                               at<int32_t>(ws, L.pos), at<int32_t>(ws, L.src), w, x_perm, sk_flags,
                               stream));
  return MOE_OK;
}

// Router stage shared by moe_route and moe_forward. Token choice writes idx/w and the
// per-block dispatch tables (the dispatch itself follows: run_dispatch_tc); expert choice
// writes idx/score and the group offsets, and with z_loss leaves the per-block z-loss
// partials in the workspace for launch_aux_final.
// select_src / sk_flags (expert choice, or nullptr): the select also writes each row's token
// and clears the GEMMs' stream-K flags, when no permute follows it.
moe_status run_router(const moe_shape& s, const Layout& L, const void* x, const void* W_g,
                      const float* b_g, const moe_noise* noise, int32_t* idx, float* w,
                      float* probs, int32_t* user_counts, float* z_loss, void* ws,
                      hipStream_t stream, int32_t* select_src = nullptr,
                      int32_t* sk_flags = nullptr, int32_t* ec_runs = nullptr) {
  const bool want_z = z_loss != nullptr;
  const int bf = s.dtype == MOE_BF16;
  RouterArgs a{};
  a.x = x;
  a.Wg = W_g;
  a.bias = b_g;
  a.Wn = noise ? noise->W_noise : nullptr;
  a.eps = noise ? noise->eps : nullptr;
  if (noise && !noise->eps) {  // drawn in the router kernel
    a.draw = 1;
    a.seed_lo = (uint32_t)noise->seed;
    a.seed_hi = (uint32_t)(noise->seed >> 32);
    a.off_lo = (uint32_t)noise->offset;
    a.off_hi = (uint32_t)(noise->offset >> 32);
    a.noise_scale = noise->scale;
  }
  a.T = (int)s.T;
  a.d = (int)s.d_model;
  a.E = s.E;
  a.k = s.k;
  a.renorm = s.renormalize;
  a.blk_zsum = want_z ? at<float>(ws, L.blk_zsum) : nullptr;
  if (is_tc(s.mode)) {
    a.idx = idx;
    a.w = w;
    a.probs = probs;
    a.lrank = at<int32_t>(ws, L.lrank);
    a.blk_counts = at<int32_t>(ws, L.blk_counts);
    a.blk_psum = at<float>(ws, L.blk_psum);
    MOE_LAUNCH(MOE_STAGE_ROUTER, launch_router(a, bf, 0, stream));
  } else {
    a.logitsT = at<float>(ws, L.logitsT);
    MOE_LAUNCH(MOE_STAGE_ROUTER, launch_router(a, bf, 1, stream));
    MOE_LAUNCH(MOE_STAGE_EC_SELECT,
               launch_ec_select(at<float>(ws, L.logitsT), (int)s.T, s.E, (int)L.C, idx, w, probs,
                                at<int32_t>(ws, L.offsets), user_counts, select_src, sk_flags,
                                ec_runs, stream));
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int32_t status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL_ARG: return "a required pointer is NULL";
    case MOE_ERR_BAD_SHAPE: return "sizes out of range or inconsistent";
    case MOE_ERR_UNSUPPORTED: return "request not supported by this library";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than moe_workspace_size()";
    case MOE_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case MOE_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

moe_status moe_capacity(const moe_shape* shape, int64_t* capacity) {
  if (!shape || !capacity) return MOE_ERR_NULL_ARG;
  if (shape->mode != MOE_EXPERT_CHOICE && shape->mode != MOE_TOKEN_CHOICE_CAPACITY)
    return MOE_ERR_BAD_SHAPE;
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  *capacity = shape->mode == MOE_EXPERT_CHOICE ? ec_capacity(*shape) : tc_capacity(*shape);
  return MOE_OK;
}

moe_status moe_workspace_size(const moe_shape* shape, size_t* bytes) {
  if (!bytes) return MOE_ERR_NULL_ARG;
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  *bytes = make_layout(*shape).total;
  return MOE_OK;
}

moe_status moe_workspace_offset(const moe_shape* shape, int32_t which, size_t* offset) {
  if (!offset) return MOE_ERR_NULL_ARG;
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  const Layout L = make_layout(*shape);
  switch (which) {
    case MOE_WS_OFFSETS: *offset = L.offsets; return MOE_OK;
    case MOE_WS_POS:
      if (!is_tc(shape->mode)) return MOE_ERR_UNSUPPORTED;
      *offset = L.pos;
      return MOE_OK;
    case MOE_WS_SRC: *offset = L.src; return MOE_OK;
    case MOE_WS_XPERM:
      if (!L.xperm) return MOE_ERR_UNSUPPORTED;
      *offset = L.x_perm;
      return MOE_OK;
    case MOE_WS_H: *offset = L.h; return MOE_OK;
    case MOE_WS_O: *offset = L.o; return MOE_OK;
    default: return MOE_ERR_BAD_SHAPE;
  }
}

moe_status moe_route(const moe_shape* shape, const void* x, const void* W_g, const float* b_g,
                     const moe_noise* noise, int32_t* idx, float* w, float* probs,
                     int32_t* counts, float* z_loss, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  st = check_noise(s, noise);
  if (st != MOE_OK) return st;
  if (s.T > 0 && (!idx || !w || !x || !W_g || !ws)) return MOE_ERR_NULL_ARG;
  if (!aligned16(x) || !aligned16(W_g) || !aligned16(ws)) return MOE_ERR_MISALIGNED;
  const Layout L = make_layout(s);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (s.T == 0) return zero_stats(s.E, nullptr, nullptr, nullptr, counts, z_loss, stream);
  st = run_router(s, L, x, W_g, b_g, noise, idx, w, probs, counts, z_loss, ws, stream);
  if (st != MOE_OK) return st;
  if (!is_tc(s.mode)) {
    if (z_loss)
      MOE_LAUNCH(MOE_STAGE_AUX, launch_aux_final(nullptr, nullptr, L.nblk, (int)s.T, 0, s.k,
                                                 nullptr, nullptr, nullptr, nullptr,
                                                 at<float>(ws, L.blk_zsum), z_loss, stream));
    return MOE_OK;
  }
  // counts and z_loss; with a capacity the dispatch also decides which slots stay (weights
  // only, no row copies)
  return run_dispatch_tc(s, L, x, idx, w, counts, nullptr, nullptr, nullptr, z_loss, nullptr,
                         nullptr, s.mode == MOE_TOKEN_CHOICE_CAPACITY, ws, stream);
}

}  // extern "C"

// Every host check of moe_forward except those of the workspace; *ws_need gets the
// workspace size the shape needs. Shared with the allocation-free entry point.
moe_status forward_host_checks(const moe_shape* shape, const void* x, const void* W_g,
                               const moe_noise* noise, const void* W_gate, const void* W_up,
                               const void* W_down, const float* y, const float* f,
                               const float* p, const float* loss, size_t* ws_need) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  if (s.mode == MOE_EXPERT_CHOICE && (f || p || loss)) return MOE_ERR_UNSUPPORTED;
  st = check_noise(s, noise);
  if (st != MOE_OK) return st;
  if (s.T > 0 && (!x || !W_g || !W_gate || !W_up || !W_down || !y)) return MOE_ERR_NULL_ARG;
  if (!aligned16(x) || !aligned16(W_g) || !aligned16(W_gate) || !aligned16(W_up) ||
      !aligned16(W_down) || !aligned16(y))
    return MOE_ERR_MISALIGNED;
  *ws_need = make_layout(s).total;
  return MOE_OK;
}

extern "C" {

moe_status moe_forward(const moe_shape* shape, const void* x, const void* W_g, const float* b_g,
                       const moe_noise* noise, const void* W_gate, const void* W_up,
                       const void* W_down, float* y,
                       int32_t* idx, float* w, float* probs, int32_t* counts, float* f, float* p,
                       float* loss, float* z_loss, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  size_t need = 0;
  moe_status st = forward_host_checks(shape, x, W_g, noise, W_gate, W_up, W_down, y, f, p, loss,
                                      &need);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  if (s.T > 0 && !ws) return MOE_ERR_NULL_ARG;
  if (!aligned16(ws)) return MOE_ERR_MISALIGNED;
  if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  const Layout L = make_layout(s);
  if (s.T == 0) return zero_stats(s.E, f, p, loss, counts, z_loss, stream);

  const int bf = s.dtype == MOE_BF16;
  const int eb = bf ? 2 : 4;
  const int T = (int)s.T, d = (int)s.d_model, ff = (int)s.d_ff, E = s.E;
  const int R = (int)L.R;
  int32_t* idx_b = idx ? idx : at<int32_t>(ws, L.idx);
  float* w_b = w ? w : at<float>(ws, L.w);
  const int32_t* offsets = at<int32_t>(ws, L.offsets);
  void* h_lo = L.h_lo ? at<void>(ws, L.h_lo) : nullptr;

  void* x_perm = L.xperm ? at<void>(ws, L.x_perm) : nullptr;  // nullptr: no row copies
  int32_t* src = at<int32_t>(ws, L.src);
  const StreamK sk{L.stream_k ? at<float>(ws, L.sk_partial) : nullptr,
                   L.stream_k ? at<int32_t>(ws, L.sk_flags) : nullptr};
  // expert choice without row copies: the select writes each row's token and clears the
  // stream-K flags itself, and no permute runs
  const bool ec_direct = !is_tc(s.mode) && !x_perm;
  int32_t* ec_runs = is_tc(s.mode) ? nullptr : at<int32_t>(ws, L.ec_runs);
  st = run_router(s, L, x, W_g, b_g, noise, idx_b, w_b, probs, counts, z_loss, ws, stream,
                  ec_direct ? src : nullptr, ec_direct ? sk.flags : nullptr, ec_runs);
  if (st != MOE_OK) return st;
  if (is_tc(s.mode)) {
    st = run_dispatch_tc(s, L, x, idx_b, w_b, counts, f, p, loss, z_loss, x_perm, sk.flags, true,
                         ws, stream);
    if (st != MOE_OK) return st;
  } else if (!ec_direct) {
    MOE_LAUNCH(MOE_STAGE_PERMUTE, launch_permute_ec(x, eb, d, E, (int)L.C, idx_b, src, x_perm,
                                                    sk.flags, stream));
  }
  MOE_LAUNCH(MOE_STAGE_GEMM_GATE_UP,
             launch_gemm_gateup(bf, x_perm ? x_perm : x, x_perm ? nullptr : src, W_gate, W_up,
                                offsets, E, R, d, ff, at<void>(ws, L.h), h_lo, sk, stream));
  MOE_LAUNCH(MOE_STAGE_GEMM_DOWN,
             launch_gemm_down(bf, at<void>(ws, L.h), W_down, offsets, E, R, ff, d,
                              at<float>(ws, L.o), h_lo ? R : 0, sk, stream));
  if (is_tc(s.mode)) {
    MOE_LAUNCH(MOE_STAGE_COMBINE, launch_combine_tc(at<float>(ws, L.o), at<int32_t>(ws, L.pos),
                                                    w_b, T, d, s.k, y, stream));
    // (f, p, loss and z_loss came out of the dispatch scan)
  } else {
    MOE_LAUNCH(MOE_STAGE_COMBINE, launch_combine_ec(at<float>(ws, L.o), idx_b, w_b, ec_runs, T, d, E,
                                                    (int)L.C, y, stream));
    if (z_loss)
      MOE_LAUNCH(MOE_STAGE_AUX, launch_aux_final(nullptr, nullptr, L.nblk, T, 0, s.k, nullptr,
                                                 nullptr, nullptr, nullptr,
                                                 at<float>(ws, L.blk_zsum), z_loss, stream));
  }
  return MOE_OK;
}

moe_status moe_aux_loss(const moe_shape* shape, const float* probs, const int32_t* idx, float* f,
                        float* p, float* loss, int32_t* counts, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  if (!is_tc(s.mode)) return MOE_ERR_UNSUPPORTED;
  if (!f || !p || !loss) return MOE_ERR_NULL_ARG;
  if (s.T > 0 && (!probs || !idx || !ws)) return MOE_ERR_NULL_ARG;
  if (!aligned16(ws)) return MOE_ERR_MISALIGNED;
  const Layout L = make_layout(s);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (s.T == 0) return zero_stats(s.E, f, p, loss, counts, nullptr, stream);
  MOE_LAUNCH(MOE_STAGE_AUX, launch_aux_partials(probs, idx, (int)s.T, s.E, s.k,
                                                at<int32_t>(ws, L.blk_counts),
                                                at<float>(ws, L.blk_psum), stream));
  MOE_LAUNCH(MOE_STAGE_AUX, launch_aux_final(at<int32_t>(ws, L.blk_counts), at<float>(ws, L.blk_psum),
                                             L.nblk, (int)s.T, s.E, s.k, f, p, loss, counts,
                                             nullptr, nullptr, stream));
  return MOE_OK;
}

moe_status moe_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  g_prof_on = on != 0;
  return MOE_OK;
}

moe_status moe_profile_read(double* total_ms, int64_t* launches, int32_t n) {
  if (n < 0) return MOE_ERR_BAD_SHAPE;
  if (n > 0 && (!total_ms || !launches)) return MOE_ERR_NULL_ARG;
  std::lock_guard<std::mutex> g(g_prof_mu);
  for (int i = 0; i < n; ++i) {
    total_ms[i] = 0.0;
    launches[i] = 0;
  }
  moe_status st = MOE_OK;
  for (const ProfRec& r : g_prof_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      st = MOE_ERR_HIP;
    if (r.stage >= 0 && r.stage < n) {
      total_ms[r.stage] += ms;
      launches[r.stage] += 1;
    }
    g_event_pool.push_back(r.a);
    g_event_pool.push_back(r.b);
  }
  g_prof_recs.clear();
  return st;
}

const char* moe_stage_name(int32_t stage) {
  static const char* names[MOE_NUM_STAGES] = {"router", "dispatch_scan", "permute",
                                               "gemm_gate_up", "gemm_down", "combine",
                                               "aux", "ec_select"};
  if (stage < 0 || stage >= MOE_NUM_STAGES) return "unknown";
  return names[stage];
}

}  // extern "C"
