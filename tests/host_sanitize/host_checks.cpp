// Drives the host side of the C ABI (csrc/moe_api.hip, built with AddressSanitizer and
// UndefinedBehaviorSanitizer and linked against the stand-ins of stub_kernels.cpp) through
// every argument error and a sweep of extreme shapes: 64-bit size arithmetic on
// caller-controlled sizes (workspace layout, capacities) must neither overflow nor index
// outside the workspace. Runs without a GPU. Exit status 0 and a final "passed" line when
// every check holds; a sanitizer report aborts the run.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "moe.h"
#include "stub_control.h"

static int failures = 0;
static long checks = 0;

static void check(bool cond, const char* what, long a = 0) {
  ++checks;
  if (!cond) {
    ++failures;
    printf("FAIL %s (%ld)\n", what, a);
  }
}

static moe_shape shape(int64_t T, int64_t d, int64_t f, int32_t E, int32_t k, int32_t mode,
                       int32_t dtype, double cf) {
  moe_shape s;
  memset(&s, 0, sizeof s);
  s.T = T;
  s.d_model = d;
  s.d_ff = f;
  s.E = E;
  s.k = k;
  s.mode = mode;
  s.dtype = dtype;
  s.renormalize = 1;
  s.capacity_factor = cf;
  return s;
}

// A fake device address range for the workspace: never dereferenced (the stand-ins only
// compare addresses), placed high so that offsets of terabytes do not wrap.
static void* const kWs = reinterpret_cast<void*>(uintptr_t(1) << 44);
static void* const kP = reinterpret_cast<void*>(uintptr_t(1) << 46);  // other buffers

// Every entry point on one shape, with a workspace of exactly the reported size.
static void run_all(const moe_shape& s) {
  size_t ws = 0;
  const moe_status st = moe_workspace_size(&s, &ws);
  int64_t cap = 0;
  moe_capacity(&s, &cap);
  for (int which = -1; which <= 6; ++which) {
    size_t off = 0;
    // (a buffer of no elements, e.g. with T = 0, may sit at the very end)
    if (moe_workspace_offset(&s, which, &off) == MOE_OK)
      check(off <= ws && off % 256 == 0, "offset inside the workspace", which);
  }
  if (st != MOE_OK) {
    // a shape the size check refuses must be refused by every entry point, before any launch
    const long before = stub_launches();
    float* fp = static_cast<float*>(kP);
    int32_t* ip = static_cast<int32_t*>(kP);
    check(moe_forward(&s, kP, kP, nullptr, nullptr, kP, kP, kP, fp, nullptr, nullptr, nullptr,
                      nullptr, nullptr, nullptr, nullptr, nullptr, kWs, (size_t)1 << 40,
                      nullptr) == st,
          "forward refuses the shape", st);
    check(moe_route(&s, kP, kP, nullptr, nullptr, ip, fp, nullptr, nullptr, nullptr, kWs,
                    (size_t)1 << 40, nullptr) == st,
          "route refuses the shape", st);
    check(stub_launches() == before, "nothing launched for a refused shape");
    return;
  }
  stub_set_workspace(kWs, ws);
  float* fp = static_cast<float*>(kP);
  int32_t* ip = static_cast<int32_t*>(kP);
  const bool tc = s.mode != MOE_EXPERT_CHOICE;
  moe_status r = moe_forward(&s, kP, kP, fp, nullptr, kP, kP, kP, fp, ip, fp, fp, ip,
                             tc ? fp : nullptr, tc ? fp : nullptr, tc ? fp : nullptr, fp, kWs, ws,
                             nullptr);
  check(r == MOE_OK, "forward on a valid shape", r);
  r = moe_forward(&s, kP, kP, nullptr, nullptr, kP, kP, kP, fp, nullptr, nullptr, nullptr,
                  nullptr, nullptr, nullptr, nullptr, nullptr, kWs, ws, nullptr);
  check(r == MOE_OK, "forward with only y", r);
  r = moe_route(&s, kP, kP, nullptr, nullptr, ip, fp, fp, ip, fp, kWs, ws, nullptr);
  check(r == MOE_OK, "route on a valid shape", r);
  if (tc) {
    moe_noise nz = {kP, fp, 0, 0, 0.f};
    r = moe_route(&s, kP, kP, nullptr, &nz, ip, fp, nullptr, nullptr, nullptr, kWs, ws, nullptr);
    check(r == MOE_OK, "noisy route", r);
    moe_noise nzd = {kP, nullptr, ~0ull, 1ull << 40, 0.5f};
    r = moe_route(&s, kP, kP, nullptr, &nzd, ip, fp, nullptr, nullptr, nullptr, kWs, ws, nullptr);
    check(r == MOE_OK, "noisy route, draw in the kernel", r);
    r = moe_aux_loss(&s, fp, ip, fp, fp, fp, ip, kWs, ws, nullptr);
    check(r == MOE_OK, "aux loss on a valid shape", r);
  }
  check(moe_forward(&s, kP, kP, nullptr, nullptr, kP, kP, kP, fp, nullptr, nullptr, nullptr,
                    nullptr, nullptr, nullptr, nullptr, nullptr, kWs, ws - 1, nullptr) ==
            (s.T == 0 && ws == 0 ? MOE_OK : MOE_ERR_WORKSPACE_TOO_SMALL),
        "workspace one byte short");
  stub_set_workspace(nullptr, 0);
}

int main() {
  const int32_t modes[] = {MOE_TOKEN_CHOICE, MOE_EXPERT_CHOICE, MOE_TOKEN_CHOICE_CAPACITY};
  const int32_t dtypes[] = {MOE_FP32, MOE_BF16};
  const int64_t Ts[] = {0, 1, 63, 64, 65, 4096, 16384, (1ll << 28) + 3, (1ll << 31) / 8 - 1,
                        (1ll << 31) - 1, 1ll << 31, (1ll << 40), -1, INT64_MAX};
  const int64_t dims[] = {64, 128, 4096, 14336, 1 << 20, (1 << 20) + 64, 0, 72, -64,
                          INT64_MAX};
  const int32_t Es[] = {1, 8, 16, 64, 65, 0, -3};
  const int32_t ks[] = {1, 2, 4, 8, 9, 0};
  const double cfs[] = {1.0, 0.7, 1e-300, 1e300, INFINITY, NAN, -1.0, 0.0};
  long shapes = 0;
  for (int32_t mode : modes)
    for (int32_t dt : dtypes)
      for (int64_t T : Ts)
        for (int64_t d : dims)
          for (int64_t f : {dims[0], dims[2], dims[4], dims[5], dims[7]})
            for (int32_t E : Es)
              for (int32_t k : ks) {
                if (mode == MOE_EXPERT_CHOICE && k != 1) continue;
                for (double cf : cfs) {
                  if (mode == MOE_TOKEN_CHOICE && cf != 1.0) continue;
                  run_all(shape(T, d, f, E, k, mode, dt, cf));
                  ++shapes;
                }
              }
  // out-of-range enum values and a renormalize flag outside {0, 1}
  for (int32_t bad : {-1, 3, 1 << 30}) {
    moe_shape s = shape(64, 64, 64, 8, 2, bad, MOE_BF16, 1.0);
    size_t ws;
    check(moe_workspace_size(&s, &ws) == MOE_ERR_BAD_SHAPE, "bad mode", bad);
    s = shape(64, 64, 64, 8, 2, MOE_TOKEN_CHOICE, bad == 3 ? 2 : bad, 1.0);
    check(moe_workspace_size(&s, &ws) == MOE_ERR_BAD_SHAPE, "bad dtype", bad);
    s = shape(64, 64, 64, 8, 2, MOE_TOKEN_CHOICE, MOE_BF16, 1.0);
    s.renormalize = bad;
    check(moe_workspace_size(&s, &ws) == MOE_ERR_BAD_SHAPE, "bad renormalize", bad);
  }
  // null arguments everywhere
  size_t ws;
  int64_t cap;
  check(moe_workspace_size(nullptr, &ws) == MOE_ERR_NULL_ARG, "null shape");
  moe_shape s = shape(64, 64, 64, 8, 2, MOE_TOKEN_CHOICE, MOE_BF16, 1.0);
  check(moe_workspace_size(&s, nullptr) == MOE_ERR_NULL_ARG, "null size");
  check(moe_capacity(&s, nullptr) == MOE_ERR_NULL_ARG, "null capacity");
  check(moe_capacity(nullptr, &cap) == MOE_ERR_NULL_ARG, "null capacity shape");
  check(moe_workspace_offset(&s, 0, nullptr) == MOE_ERR_NULL_ARG, "null offset");
  check(moe_forward(nullptr, kP, kP, nullptr, nullptr, kP, kP, kP, (float*)kP, nullptr, nullptr,
                    nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, kWs, 1, nullptr) ==
            MOE_ERR_NULL_ARG,
        "forward without a shape");
  // status strings and stage names for every value, in and out of range
  for (int32_t v : {-1000, -1, 0, 1, 2, 3, 4, 5, 6, 7, 100, INT32_MAX, INT32_MIN}) {
    check(moe_status_string(v) != nullptr && strlen(moe_status_string(v)) > 0, "status string");
    check(moe_stage_name(v) != nullptr, "stage name");
  }
  // stage timing: events that fail to create (no device), then fake events that work
  double ms[MOE_NUM_STAGES];
  int64_t n[MOE_NUM_STAGES];
  check(moe_profile_read(nullptr, nullptr, -1) == MOE_ERR_BAD_SHAPE, "negative stage count");
  check(moe_profile_read(nullptr, n, 2) == MOE_ERR_NULL_ARG, "null totals");
  moe_profile_enable(1);
  run_all(shape(1000, 256, 512, 8, 2, MOE_TOKEN_CHOICE, MOE_BF16, 1.0));
  check(moe_profile_read(ms, n, MOE_NUM_STAGES) == MOE_OK && n[0] == 0, "no events recorded");
  stub_events_work(1);
  for (int i = 0; i < 3; ++i) run_all(shape(1000, 256, 512, 8, 2, MOE_TOKEN_CHOICE, MOE_BF16, 1.0));
  check(moe_profile_read(ms, n, MOE_NUM_STAGES) == MOE_OK && n[MOE_STAGE_ROUTER] > 0 &&
            fabs(ms[MOE_STAGE_ROUTER] - 0.5 * n[MOE_STAGE_ROUTER]) < 1e-9,
        "events recorded and read");
  check(moe_profile_read(ms, n, 3) == MOE_OK && n[0] == 0, "read clears");
  moe_profile_enable(0);
  printf("shapes %ld, checks %ld, launches %ld\n", shapes, checks, stub_launches());
  printf("%s: %d failure(s)\n", failures ? "FAILED" : "passed", failures);
  return failures ? 1 : 0;
}
