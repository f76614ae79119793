/*
 * Host-side exercise of the C ABI (include/tra.h) for sanitizer builds of the
 * library: every path below runs on the host only (validation, radius
 * tables, status strings, argument checks, allocation and launch failures
 * forced through TRA_FAULT), so it needs no GPU.  Exits 0 when every call
 * returns the documented status.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tra.h"

static int failures = 0;

#define EXPECT(cond)                                                    \
  do {                                                                  \
    if (!(cond)) {                                                      \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                       \
    }                                                                   \
  } while (0)

static tra_params default_params(void) {
  tra_params p;
  memset(&p, 0, sizeof p);
  p.a = 1.0;
  p.c = -0.8125;
  p.budget_min = 16.0;
  p.budget_max = 75600.0;
  p.decay = 0.5;
  p.radius_override = -1.0;
  p.levels_per_nat = 8;
  p.pool_h = p.pool_w = 16;
  p.tile_h = p.tile_w = 8;
  p.generator = TRA_GEN_ENTROPY_DISK;
  p.vote_threshold = 1;
  p.block_mask = 0;
  return p;
}

int main(void) {
  const tra_shape wan = {1, 40, 21, 45, 80, 128, TRA_BF16};
  tra_params p = default_params();

  /* validation */
  EXPECT(tra_params_validate(&wan, &p) == TRA_OK);
  EXPECT(tra_params_validate(NULL, &p) == TRA_ERR_INVALID_ARG);
  EXPECT(tra_params_validate(&wan, NULL) == TRA_ERR_INVALID_ARG);
  tra_shape bad = wan;
  bad.head_dim = 96;
  EXPECT(tra_params_validate(&bad, &p) == TRA_ERR_DTYPE);
  bad = wan;
  bad.T = 0;
  EXPECT(tra_params_validate(&bad, &p) == TRA_ERR_SHAPE);
  tra_params bp = p;
  bp.decay = 0.0;
  EXPECT(tra_params_validate(&wan, &bp) == TRA_ERR_INVALID_ARG);
  bp = p;
  bp.generator = 7;
  EXPECT(tra_params_validate(&wan, &bp) == TRA_ERR_INVALID_ARG);
  bp = p;
  bp.regroup = 1;
  EXPECT(tra_params_validate(&wan, &bp) == TRA_OK);
  bp.block_mask = 1; /* block masks are per query tile */
  EXPECT(tra_params_validate(&wan, &bp) == TRA_ERR_INVALID_ARG);
  EXPECT(strlen(tra_last_error()) > 0);
  bp = p; /* attention groups of 2 or 3 query-tile rows; regrouping orders 2 x 2 groups */
  bp.group_rows = 3;
  EXPECT(tra_params_validate(&wan, &bp) == TRA_OK);
  bp.group_rows = 4;
  EXPECT(tra_params_validate(&wan, &bp) == TRA_ERR_INVALID_ARG);
  bp.group_rows = 3;
  bp.regroup = 1;
  EXPECT(tra_params_validate(&wan, &bp) == TRA_ERR_INVALID_ARG);
  bp.group_rows = 2;
  EXPECT(tra_params_validate(&wan, &bp) == TRA_OK);

  /* radius tables: size query, then the table */
  int32_t n_levels = 0, k_lo = 0;
  EXPECT(tra_radius_table(&wan, &p, NULL, NULL, &n_levels, &k_lo) == TRA_OK);
  EXPECT(n_levels > 0 && k_lo == 23);
  int32_t* r2 = (int32_t*)malloc(sizeof(int32_t) * (size_t)n_levels * (size_t)wan.T);
  double* r0sq = (double*)malloc(sizeof(double) * (size_t)n_levels);
  EXPECT(tra_radius_table(&wan, &p, r2, r0sq, &n_levels, &k_lo) == TRA_OK);
  for (int r = 0; r < n_levels; ++r) {
    EXPECT(r2[(size_t)r * wan.T] >= 0);           /* frame 0 is always active */
    for (int dl = 1; dl < wan.T; ++dl) EXPECT(r2[(size_t)r * wan.T + dl] <= r2[(size_t)r * wan.T + dl - 1]);
  }
  free(r2);
  free(r0sq);
  for (int gen = 1; gen <= 3; ++gen) {
    tra_params gp = p;
    gp.generator = gen;
    gp.radius_override = 9.0;
    EXPECT(tra_radius_table(&wan, &gp, NULL, NULL, &n_levels, &k_lo) == TRA_OK);
    EXPECT(n_levels == 1 && k_lo == -1);
  }

  /* status strings */
  for (int s = 0; s <= 8; ++s) EXPECT(strncmp(tra_status_string((tra_status)s), "TRA_", 4) == 0);
  EXPECT(strcmp(tra_status_string((tra_status)99), "TRA_ERR_UNKNOWN") == 0);

  /* NULL plans and pointers are rejected before any device work */
  int64_t a = 0, b = 0;
  void* fake = (void*)(uintptr_t)4096;
  EXPECT(tra_attention(NULL, fake, fake, fake, (void*)(uintptr_t)8192, NULL) == TRA_ERR_INVALID_ARG);
  EXPECT(tra_plan_stats(NULL, &a, &b, NULL) == TRA_ERR_INVALID_ARG);
  EXPECT(tra_plan_drift(NULL, fake, fake, &a, NULL) == TRA_ERR_INVALID_ARG);
  EXPECT(tra_plan_drift_noalloc(NULL, fake, fake, &a, NULL) == TRA_ERR_INVALID_ARG);
  EXPECT(tra_plan_export(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == TRA_ERR_INVALID_ARG);
  EXPECT(tra_plan_export_regroup(NULL, NULL, NULL) == TRA_ERR_INVALID_ARG);
  EXPECT(tra_plan_rebuild(NULL, fake, fake, NULL) == TRA_ERR_INVALID_ARG);
  EXPECT(tra_dense_attention(&wan, fake, fake, fake, fake, NULL, NULL) == TRA_ERR_INVALID_ARG); /* o aliases q */
  EXPECT(tra_dense_attention(&wan, (void*)(uintptr_t)4100, fake, fake, (void*)(uintptr_t)8192, NULL, NULL) ==
         TRA_ERR_INVALID_ARG); /* misaligned */
  tra_plan_destroy(NULL);
  tra_schedule_destroy(NULL);

  /* forced allocation failure: distinct status, *out NULL */
  tra_plan* plan = (tra_plan*)fake;
  setenv("TRA_FAULT", "alloc", 1);
  EXPECT(tra_plan_create(&wan, &p, fake, fake, NULL, &plan) == TRA_ERR_OOM);
  EXPECT(plan == NULL);
  plan = (tra_plan*)fake;
  EXPECT(tra_plan_create_from_entropy(&wan, &p, (const float*)fake, NULL, &plan) == TRA_ERR_OOM);
  EXPECT(plan == NULL);
  {
    /* a plan imported from levels: every level is checked first */
    const size_t nq = (size_t)wan.B * wan.heads * wan.T * wan.H * wan.W;
    int16_t* lv = (int16_t*)malloc(sizeof(int16_t) * nq);
    EXPECT(tra_radius_table(&wan, &p, NULL, NULL, &n_levels, &k_lo) == TRA_OK);
    for (size_t i = 0; i < nq; ++i) lv[i] = (int16_t)k_lo;
    plan = (tra_plan*)fake;
    EXPECT(tra_plan_import(&wan, &p, lv, NULL, NULL, NULL, &plan) == TRA_ERR_OOM);
    EXPECT(plan == NULL);
    lv[nq - 1] = (int16_t)(k_lo - 1);
    plan = (tra_plan*)fake;
    EXPECT(tra_plan_import(&wan, &p, lv, NULL, NULL, NULL, &plan) == TRA_ERR_INVALID_ARG);
    EXPECT(plan == NULL);
    EXPECT(tra_plan_import(&wan, &p, NULL, NULL, NULL, NULL, &plan) == TRA_ERR_INVALID_ARG);
    free(lv);
  }
  tra_schedule* sched = (tra_schedule*)fake;
  const tra_schedule_params sp = {2, 0, 0.1};
  EXPECT(tra_schedule_create(&wan, &p, &sp, &sched) == TRA_ERR_OOM);
  EXPECT(sched == NULL);

  /* forced launch failure: distinct status */
  setenv("TRA_FAULT", "launch:1", 1);
  EXPECT(tra_dense_attention(&wan, fake, (void*)(uintptr_t)8192, (void*)(uintptr_t)12288,
                             (void*)(uintptr_t)16384, NULL, NULL) == TRA_ERR_HIP);
  EXPECT(strstr(tra_last_error(), "injected launch failure") != NULL);

  /* malformed settings inject nothing (checked on a host-only call) */
  setenv("TRA_FAULT", "alloc:0", 1);
  EXPECT(tra_params_validate(&wan, &p) == TRA_OK);
  unsetenv("TRA_FAULT");

  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("abi host checks passed\n");
  return 0;
}
