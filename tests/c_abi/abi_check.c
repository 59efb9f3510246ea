/* A plain C11 consumer of include/moe.h: links libmoe_hip.so and exercises every entry
 * point whose checks complete on the host (sizes, capacities, workspace offsets, status
 * strings, argument errors, profiling with nothing recorded). Needs no GPU: each call
 * below returns before any HIP call. Prints one line per check; exit status 0 when all
 * pass. */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "moe.h"

static int failures = 0;

static void check(int cond, const char* what) {
  printf("%s %s\n", cond ? "ok  " : "FAIL", what);
  if (!cond) ++failures;
}

static moe_shape shape(int64_t T, int64_t d, int64_t f, int32_t E, int32_t k, int32_t mode,
                       double cf) {
  moe_shape s;
  memset(&s, 0, sizeof s);
  s.T = T;
  s.d_model = d;
  s.d_ff = f;
  s.E = E;
  s.k = k;
  s.mode = mode;
  s.dtype = MOE_BF16;
  s.renormalize = 1;
  s.capacity_factor = cf;
  return s;
}

int main(void) {
  /* status strings: never NULL, distinct for the defined codes */
  for (int c = 0; c <= MOE_ERR_HIP; ++c) check(moe_status_string(c) != NULL, "status string");
  check(strcmp(moe_status_string(MOE_OK), moe_status_string(MOE_ERR_HIP)) != 0,
        "status strings differ");
  check(moe_status_string(12345) != NULL, "unknown status string");

  /* capacities */
  int64_t cap = -1;
  moe_shape ec = shape(8192, 1024, 4096, 16, 1, MOE_EXPERT_CHOICE, 1.0);
  check(moe_capacity(&ec, &cap) == MOE_OK && cap == 512, "expert-choice capacity 8192*1/16");
  moe_shape tcc = shape(100, 64, 64, 8, 2, MOE_TOKEN_CHOICE_CAPACITY, 1.25);
  check(moe_capacity(&tcc, &cap) == MOE_OK && cap == 31, "token-choice capacity of T=100 E=8 k=2 cf=1.25");
  /* the factor is a double: 0.7 (not exact in binary) gives int(1000 * 0.7 / 10) = 70 as
     the pages' double arithmetic does; its float rounding would give 69 */
  moe_shape ec7 = shape(1000, 64, 64, 10, 1, MOE_EXPERT_CHOICE, 0.7);
  check(moe_capacity(&ec7, &cap) == MOE_OK && cap == 70, "expert-choice capacity 1000*0.7/10");
  moe_shape tc9 = shape(1000, 64, 64, 10, 2, MOE_TOKEN_CHOICE_CAPACITY, 0.9);
  check(moe_capacity(&tc9, &cap) == MOE_OK && cap == 180, "token-choice capacity 1000/10*0.9*2");
  moe_shape tc = shape(4096, 1024, 4096, 8, 2, MOE_TOKEN_CHOICE, 1.0);
  check(moe_capacity(&tc, &cap) == MOE_ERR_BAD_SHAPE, "plain token choice has no capacity");
  check(moe_capacity(NULL, &cap) == MOE_ERR_NULL_ARG, "capacity of NULL shape");

  /* workspace size and offsets */
  size_t ws = 0, off = 0;
  check(moe_workspace_size(&tc, &ws) == MOE_OK && ws > 0, "workspace size");
  check(moe_workspace_offset(&tc, MOE_WS_POS, &off) == MOE_OK && off < ws && off % 16 == 0,
        "position table inside the workspace");
  check(moe_workspace_offset(&ec, MOE_WS_POS, &off) == MOE_ERR_UNSUPPORTED,
        "no position table in expert choice");
  moe_shape bad = shape(64, 100, 64, 8, 2, MOE_TOKEN_CHOICE, 1.0); /* d_model % 64 != 0 */
  check(moe_workspace_size(&bad, &ws) == MOE_ERR_UNSUPPORTED, "d_model not a multiple of 64");
  bad = shape(64, 64, 64, 65, 2, MOE_TOKEN_CHOICE, 1.0);
  check(moe_workspace_size(&bad, &ws) != MOE_OK, "more than 64 experts");
  bad = shape(64, 64, 64, 16, 9, MOE_TOKEN_CHOICE, 1.0);
  check(moe_workspace_size(&bad, &ws) == MOE_ERR_UNSUPPORTED, "k = 9");
  bad = shape(64, 64, 64, 8, 2, MOE_TOKEN_CHOICE_CAPACITY, 0.0);
  check(moe_workspace_size(&bad, &ws) == MOE_ERR_BAD_SHAPE, "capacity factor 0");

  /* argument errors of the compute entry points (returned before any HIP call) */
  moe_shape s = shape(64, 128, 256, 8, 2, MOE_TOKEN_CHOICE, 1.0);
  size_t need = 0;
  moe_workspace_size(&s, &need);
  void* p = (void*)(uintptr_t)4096; /* never dereferenced */
  void* mis = (void*)(uintptr_t)4100;
  check(moe_forward(&s, NULL, p, NULL, NULL, p, p, p, p, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                    NULL, p, need, NULL) == MOE_ERR_NULL_ARG,
        "forward without x");
  check(moe_forward(&s, p, p, NULL, NULL, p, p, p, mis, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                    NULL, p, need, NULL) == MOE_ERR_MISALIGNED,
        "forward with a misaligned y");
  check(moe_forward(&s, p, p, NULL, NULL, p, p, p, p, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                    NULL, p, need - 1, NULL) == MOE_ERR_WORKSPACE_TOO_SMALL,
        "forward with a small workspace");
  moe_noise nz = {NULL, NULL, 1, 0, NAN};
  check(moe_route(&s, p, p, NULL, &nz, p, p, NULL, NULL, NULL, p, need, NULL) == MOE_ERR_BAD_SHAPE,
        "noise drawn in the kernel with a non-finite scale");
  moe_shape ecs = shape(64, 128, 256, 8, 1, MOE_EXPERT_CHOICE, 1.0);
  nz.eps = (const float*)p;
  check(moe_route(&ecs, p, p, NULL, &nz, p, p, NULL, NULL, NULL, p, need, NULL) ==
            MOE_ERR_UNSUPPORTED,
        "noise in expert choice");
  float* fp = (float*)p;
  check(moe_forward(&ecs, p, p, NULL, NULL, p, p, p, p, NULL, NULL, NULL, NULL, fp, NULL, NULL,
                    NULL, p, need, NULL) == MOE_ERR_UNSUPPORTED,
        "load-balancing statistics in expert choice");
  check(moe_aux_loss(&s, fp, (const int32_t*)p, NULL, fp, fp, NULL, p, need, NULL) ==
            MOE_ERR_NULL_ARG,
        "aux loss without f");

  /* the allocation-free entry point refuses a layer larger than its scratch */
  moe_shape big = shape(16384, 4096, 14336, 8, 2, MOE_TOKEN_CHOICE, 1.0);
  check(moe_workspace_size(&big, &need) == MOE_OK && need > MOE_NOALLOC_SCRATCH_BYTES,
        "Mixtral-size workspace exceeds the fixed scratch");
  check(moe_forward_noalloc(&big, p, p, NULL, NULL, p, p, p, p, NULL, NULL, NULL, NULL, NULL,
                            NULL, NULL, NULL, NULL) == MOE_ERR_WORKSPACE_TOO_SMALL,
        "allocation-free forward refuses a layer larger than its scratch");
  check(moe_forward_noalloc(&s, NULL, p, NULL, NULL, p, p, p, p, NULL, NULL, NULL, NULL, NULL,
                            NULL, NULL, NULL, NULL) == MOE_ERR_NULL_ARG,
        "allocation-free forward without x");

  /* profiling with nothing recorded */
  double ms[MOE_NUM_STAGES];
  int64_t n[MOE_NUM_STAGES];
  check(moe_profile_enable(0) == MOE_OK, "profiling off");
  check(moe_profile_read(ms, n, MOE_NUM_STAGES) == MOE_OK && n[0] == 0 && ms[0] == 0.0,
        "empty profile");
  check(strcmp(moe_stage_name(MOE_STAGE_GEMM_GATE_UP), "gemm_gate_up") == 0, "stage name");

  printf("%s: %d failure(s)\n", failures ? "FAILED" : "passed", failures);
  return failures ? 1 : 0;
}
