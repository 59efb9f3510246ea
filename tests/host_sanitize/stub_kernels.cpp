// Host-only stand-ins for the launch wrappers of csrc/kernels.h and the few HIP runtime
// calls the host code makes, so that csrc/moe_api.hip (argument checks, workspace layout,
// launch sequence) can be built with AddressSanitizer and UndefinedBehaviorSanitizer and
// run on a machine without a GPU. Nothing here launches or dereferences device memory.
//
// Each stand-in checks the buffers the host code hands it: a pointer that falls inside the
// caller's workspace must have its whole extent (computed from the same sizes the kernel
// would use) inside the workspace too. A violation aborts with a message.
#include <stdio.h>
#include <stdlib.h>

#include "kernels.h"
#include "stub_control.h"

namespace {
const char* g_ws_lo = nullptr;
const char* g_ws_hi = nullptr;
long g_launches = 0;
bool g_events_work = false;
long g_fake_event = 0;

void inside(const void* p, size_t bytes, const char* what) {
  const char* c = static_cast<const char*>(p);
  if (!c || !g_ws_lo || c < g_ws_lo || c >= g_ws_hi) return;  // not a workspace buffer
  if (bytes > (size_t)(g_ws_hi - c)) {
    fprintf(stderr, "workspace overflow: %s needs %zu bytes at offset %zu of %zu\n", what, bytes,
            (size_t)(c - g_ws_lo), (size_t)(g_ws_hi - g_ws_lo));
    abort();
  }
}
}  // namespace

void stub_set_workspace(const void* ws, size_t bytes) {
  g_ws_lo = static_cast<const char*>(ws);
  g_ws_hi = g_ws_lo ? g_ws_lo + bytes : nullptr;
}
long stub_launches() { return g_launches; }
void stub_events_work(int on) { g_events_work = on != 0; }

hipError_t launch_router(const RouterArgs& a, int bf16, int ec, hipStream_t) {
  ++g_launches;
  const size_t T = (size_t)a.T, k = (size_t)a.k, E = (size_t)a.E, nblk = (T + 63) / 64;
  if (!ec) {
    inside(a.idx, T * k * 4, "router idx");
    inside(a.w, T * k * 4, "router w");
    inside(a.lrank, T * k * 4, "router slot ranks");
    inside(a.blk_counts, nblk * E * 4, "router block counts");
    inside(a.blk_psum, nblk * E * 4, "router block sums");
  } else {
    inside(a.logitsT, E * T * 4, "router logits");
  }
  inside(a.blk_zsum, nblk * 4, "router z partials");
  (void)bf16;
  return hipSuccess;
}

hipError_t launch_ec_select(const float* logitsT, int T, int E, int C, int32_t* idx, float* score,
                            float* probs, int32_t* offsets, int32_t* counts, int32_t* src,
                            int32_t* sk_flags, int32_t* runs, hipStream_t) {
  ++g_launches;
  inside(logitsT, (size_t)E * T * 4, "select logits");
  inside(runs, (size_t)E * ec_run_stride(T) * 4, "select run table");
  inside(idx, (size_t)E * C * 4, "select idx");
  inside(src, (size_t)E * C * 4, "select src");
  inside(sk_flags, (size_t)kStreamKSlots * 4, "select stream-K flags");
  inside(score, (size_t)E * C * 4, "select scores");
  inside(offsets, (size_t)(E + 1) * 4, "select offsets");
  (void)probs;
  (void)counts;
  return hipSuccess;
}

hipError_t launch_dispatch_scan(const ScanArgs& a, hipStream_t) {
  ++g_launches;
  inside(a.blk_counts, (size_t)a.nblk * a.E * 4, "scan block counts");
  inside(a.counts, (size_t)a.E * 4, "scan counts");
  inside(a.offsets, (size_t)(a.E + 1) * 4, "scan offsets");
  inside(a.base, (size_t)a.nblk * a.E * 4, "scan bases");
  inside(a.blk_psum, (size_t)a.nblk * a.E * 4, "scan block sums");
  return hipSuccess;
}

hipError_t launch_dispatch_tc(const DispatchArgs& a, hipStream_t) {
  ++g_launches;
  const size_t R = (size_t)a.T * a.k;
  inside(a.lrank, R * 4, "dispatch slot ranks");
  inside(a.blk_counts, (size_t)a.nblk * a.E * 4, "dispatch block counts");
  inside(a.pos, R * 4, "dispatch pos");
  inside(a.src, R * 4, "dispatch src");
  inside(a.x_perm, R * a.d * a.elt_bytes, "dispatch rows");
  inside(a.offsets, (size_t)(a.E + 1) * 4, "dispatch offsets");
  inside(a.counts, (size_t)a.E * 4, "dispatch counts");
  inside(a.blk_psum, (size_t)a.nblk * a.E * 4, "dispatch block sums");
  inside(a.blk_zsum, (size_t)a.nblk * 4, "dispatch z partials");
  inside(a.sk_flags, kStreamKSlots * 4, "stream-K flags");
  if (a.nblk > kFusedMaxBlocks) {
    fprintf(stderr, "fused dispatch launched with %d blocks\n", a.nblk);
    abort();
  }
  return hipSuccess;
}

hipError_t launch_permute_tc(const void* x, int elt_bytes, int T, int d, int E, int k,
                             const int32_t* idx, const int32_t* lrank, const int32_t* base,
                             const int32_t* offsets, int cap, int renorm, int32_t* pos,
                             int32_t* src, float* w, void* x_perm, int32_t* sk_flags,
                             hipStream_t) {
  ++g_launches;
  const size_t R = (size_t)T * k;
  inside(pos, R * 4, "permute pos");
  inside(src, R * 4, "permute src");
  inside(x_perm, R * d * elt_bytes, "permute rows");
  inside(sk_flags, kStreamKSlots * 4, "stream-K flags");
  (void)x, (void)E, (void)idx, (void)lrank, (void)base, (void)offsets, (void)cap, (void)renorm,
      (void)w;
  return hipSuccess;
}

hipError_t launch_permute_ec(const void* x, int elt_bytes, int d, int E, int C,
                             const int32_t* idx, int32_t* src, void* x_perm, int32_t* sk_flags,
                             hipStream_t) {
  ++g_launches;
  const size_t R = (size_t)E * C;
  inside(idx, R * 4, "permute idx");
  inside(src, R * 4, "permute src");
  inside(x_perm, R * d * elt_bytes, "permute rows");
  inside(sk_flags, kStreamKSlots * 4, "stream-K flags");
  (void)x;
  return hipSuccess;
}

hipError_t launch_gemm_gateup(int bf16, const void* xp, const int32_t* gather, const void* Wgate,
                              const void* Wup, const int32_t* offsets, int E, int R_max, int d,
                              int f, void* h, void* h_lo, const StreamK& sk, hipStream_t) {
  ++g_launches;
  const size_t eb = bf16 ? 2 : 4;
  inside(xp, (size_t)R_max * d * eb, "gate/up rows");
  inside(gather, (size_t)R_max * 4, "gate/up gather");
  inside(offsets, (size_t)(E + 1) * 4, "gate/up offsets");
  inside(h, (size_t)R_max * f * eb, "gate/up h");
  inside(h_lo, (size_t)R_max * f * eb, "gate/up h residual");
  inside(sk.partial, kStreamKSlots * kStreamKSlotBytes, "stream-K partials");
  inside(sk.flags, kStreamKSlots * 4, "stream-K flags");
  (void)Wgate, (void)Wup;
  return hipSuccess;
}

hipError_t launch_gemm_down(int bf16, const void* h, const void* Wdown, const int32_t* offsets,
                            int E, int R_max, int f, int d, float* o, int lo_rows,
                            const StreamK& sk, hipStream_t) {
  ++g_launches;
  const size_t eb = bf16 ? 2 : 4;
  // with residual rows the h rows run to R_max + lo_rows
  inside(h, ((size_t)R_max + (size_t)lo_rows) * f * eb, "down h");
  inside(offsets, (size_t)(E + 1) * 4, "down offsets");
  inside(o, (size_t)R_max * d * 4, "down o");
  inside(sk.partial, kStreamKSlots * kStreamKSlotBytes, "stream-K partials");
  inside(sk.flags, kStreamKSlots * 4, "stream-K flags");
  (void)Wdown;
  return hipSuccess;
}

hipError_t launch_combine_tc(const float* o, const int32_t* pos, const float* w, int T, int d,
                             int k, float* y, hipStream_t) {
  ++g_launches;
  inside(o, (size_t)T * k * d * 4, "combine o");
  inside(pos, (size_t)T * k * 4, "combine pos");
  inside(w, (size_t)T * k * 4, "combine w");
  (void)y;
  return hipSuccess;
}

hipError_t launch_combine_ec(const float* o, const int32_t* idx, const float* score,
                             const int32_t* runs, int T, int d, int E, int C, float* y,
                             hipStream_t) {
  ++g_launches;
  inside(runs, (size_t)E * ec_run_stride(T) * 4, "combine run table");
  inside(o, (size_t)E * C * d * 4, "combine o");
  inside(idx, (size_t)E * C * 4, "combine idx");
  inside(score, (size_t)E * C * 4, "combine scores");
  (void)T, (void)y;
  return hipSuccess;
}

hipError_t launch_aux_partials(const float* probs, const int32_t* idx, int T, int E, int k,
                               int32_t* blk_counts, float* blk_psum, hipStream_t) {
  ++g_launches;
  const size_t nblk = ((size_t)T + 63) / 64;
  inside(blk_counts, nblk * E * 4, "aux block counts");
  inside(blk_psum, nblk * E * 4, "aux block sums");
  (void)probs, (void)idx, (void)k;
  return hipSuccess;
}

hipError_t launch_aux_final(const int32_t* blk_counts, const float* blk_psum, int nblk, int T,
                            int E, int k, float* f, float* p, float* loss, int32_t* counts,
                            const float* blk_zsum, float* z_loss, hipStream_t) {
  ++g_launches;
  inside(blk_counts, (size_t)nblk * E * 4, "final block counts");
  inside(blk_psum, (size_t)nblk * E * 4, "final block sums");
  inside(blk_zsum, (size_t)nblk * 4, "final z partials");
  (void)T, (void)k, (void)f, (void)p, (void)loss, (void)counts, (void)z_loss;
  return hipSuccess;
}

hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t) {
  ++g_launches;
  inside(ptr, bytes, "fill");
  return hipSuccess;
}

// The HIP runtime calls of the host code's stage timing. Without `stub_events_work` event
// creation fails (as without a device), which the timer must survive; with it, events are
// distinct fake handles that record and read back 0.5 ms.
extern "C" {
hipError_t hipEventCreate(hipEvent_t* e) {
  if (!g_events_work) return hipErrorNoDevice;
  *e = reinterpret_cast<hipEvent_t>(++g_fake_event * 64);
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
  *ms = 0.5f;
  return hipSuccess;
}
}
