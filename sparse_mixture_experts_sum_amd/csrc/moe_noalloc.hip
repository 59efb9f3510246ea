// moe_forward_noalloc: the layer forward for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
// Its workspace is `scratch`, a file-scope device array of MOE_NOALLOC_SCRATCH_BYTES that
// every GPU the library runs on holds until the process ends. The kernels are those of
// moe_forward; only where the workspace comes from differs.
//
// In host code `scratch` names a host-side stand-in, not device memory: its device address
// is looked up once per device with hipGetSymbolAddress (with that device current) and
// kept; that address, never the array's name, is what reaches the kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "api_internal.h"
#include "moe.h"

namespace {

static __device__ __attribute__((aligned(256))) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up on the first call on that device).
moe_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_forward_noalloc(const moe_shape* shape, const void* x, const void* W_g,
                                          const float* b_g, const moe_noise* noise,
                                          const void* W_gate, const void* W_up,
                                          const void* W_down, float* y, int32_t* idx, float* w,
                                          float* probs, int32_t* counts, float* f, float* p,
                                          float* loss, float* z_loss, hipStream_t stream) {
  size_t need = 0;
  moe_status st = forward_host_checks(shape, x, W_g, noise, W_gate, W_up, W_down, y, f, p, loss,
                                      &need);
  if (st != MOE_OK) return st;
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != MOE_OK) return st;
  return moe_forward(shape, x, W_g, b_g, noise, W_gate, W_up, W_down, y, idx, w, probs, counts, f,
                     p, loss, z_loss, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}
