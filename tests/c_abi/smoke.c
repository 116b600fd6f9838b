/* A plain C consumer of the C ABI (include/moonep.h): no Python, no torch.
 *
 *   smoke host   host-only calls: moonep_query, argument errors, moonep_strerror
 *   smoke gpu    plan -> dispatch -> combine -> status on the GPU, checked exactly:
 *                token t routes to experts (t + k*step) % E, all weights 1/K with K a power
 *                of two, and x holds small integers, so every dispatched row equals x[t]
 *                and every combined row equals x[t] exactly in bf16.
 * Exit status 0 on success; the first failed check is printed. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moonep.h"

#define CHECK(cond, ...)                                   \
  do {                                                     \
    if (!(cond)) {                                         \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                        \
      fprintf(stderr, "\n");                               \
      return 1;                                            \
    }                                                      \
  } while (0)

#define HIPOK(call) CHECK((call) == hipSuccess, "%s", #call)

static uint16_t bf16_of_small_int(int v) {  /* exact for |v| <= 256 */
  float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static int host_checks(void) {
  moonep_sizes s;
  CHECK(moonep_query(8, 256, 8, 4096, 32, &s) == MOONEP_OK, "query dsv3");
  CHECK(s.NvS == 33728 && s.recv_rows == 8LL * 33728 && s.T == 32768 && s.A == 262144,
        "dsv3 sizes: NvS %d", s.NvS);
  CHECK(s.plan_bytes > 0 && s.workspace_bytes > 0, "plan/workspace bytes");
  CHECK(moonep_query(3, 16, 2, 4, 4, &s) == MOONEP_EINVAL, "E %% R");
  CHECK(moonep_query(65, 65, 2, 4, 4, &s) == MOONEP_ELIMIT, "R > 64");
  CHECK(moonep_query(4, 16, 2, 4, 4, NULL) == MOONEP_EINVAL, "null out");
  moonep_plan_desc d;
  memset(&d, 0, sizeof(d));
  CHECK(moonep_dispatch(&d, NULL, 16, NULL, 0) == MOONEP_EPLAN, "uninitialised plan");
  CHECK(strcmp(moonep_strerror(MOONEP_OK), "ok") == 0, "strerror");
  printf("host checks ok\n");
  return 0;
}

static int gpu_run(void) {
  const int R = 4, E = 16, K = 2, S = 96, slots = 4, H = 64;
  moonep_sizes s;
  CHECK(moonep_query(R, E, K, S, slots, &s) == MOONEP_OK, "query");
  const int T = R * S;
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * T * K);
  float* w = (float*)malloc(sizeof(float) * T * K);
  uint16_t* x = (uint16_t*)malloc(sizeof(uint16_t) * T * H);
  uint16_t* out = (uint16_t*)malloc(sizeof(uint16_t) * T * H);
  int32_t* dst = (int32_t*)malloc(sizeof(int32_t) * T * K);
  uint16_t* row = (uint16_t*)malloc(sizeof(uint16_t) * H);
  for (int t = 0; t < T; ++t) {
    /* skewed: expert 0 and 1 take most assignments, so replicas are needed */
    for (int k = 0; k < K; ++k) {
      ids[t * K + k] = (t % 3 == 0) ? (t + k * 5) % E : k;
      w[t * K + k] = 1.0f / K;
    }
    for (int h = 0; h < H; ++h) x[t * H + h] = bf16_of_small_int(((t * 7 + h) % 33) - 16);
  }
  void *d_ids, *d_w, *d_plan, *d_ws, *d_x, *d_recv, *d_out;
  HIPOK(hipMalloc(&d_ids, sizeof(int32_t) * T * K));
  HIPOK(hipMalloc(&d_w, sizeof(float) * T * K));
  HIPOK(hipMalloc(&d_plan, (size_t)s.plan_bytes));
  HIPOK(hipMalloc(&d_ws, (size_t)s.workspace_bytes));
  HIPOK(hipMemset(d_ws, 0, (size_t)s.workspace_bytes));   /* zero before its first use */
  HIPOK(hipMalloc(&d_x, sizeof(uint16_t) * T * H));
  HIPOK(hipMalloc(&d_recv, sizeof(uint16_t) * (size_t)s.recv_rows * H));
  HIPOK(hipMalloc(&d_out, sizeof(uint16_t) * T * H));
  HIPOK(hipMemcpy(d_ids, ids, sizeof(int32_t) * T * K, hipMemcpyHostToDevice));
  HIPOK(hipMemcpy(d_w, w, sizeof(float) * T * K, hipMemcpyHostToDevice));
  HIPOK(hipMemcpy(d_x, x, sizeof(uint16_t) * T * H, hipMemcpyHostToDevice));
  hipStream_t st;
  HIPOK(hipStreamCreate(&st));
  moonep_plan_desc plan;
  int rc = moonep_plan((const int32_t*)d_ids, (const float*)d_w, R, E, K, S, slots, d_plan, d_ws,
                       &plan, st);
  CHECK(rc == MOONEP_OK, "plan: %s", moonep_strerror(rc));
  rc = moonep_dispatch(&plan, (const uint16_t*)d_x, H, (uint16_t*)d_recv, st);
  CHECK(rc == MOONEP_OK, "dispatch: %s", moonep_strerror(rc));
  rc = moonep_combine(&plan, (const uint16_t*)d_recv, H, (uint16_t*)d_out, st);
  CHECK(rc == MOONEP_OK, "combine: %s", moonep_strerror(rc));
  moonep_plan_stats stats;
  rc = moonep_plan_status(&plan, &stats, st);
  CHECK(rc == MOONEP_OK && stats.status == 0, "status %d", stats.status);
  CHECK(stats.n_replicas + stats.n_fallback > 0, "the skewed routing should need replicas");
  HIPOK(hipMemcpy(out, d_out, sizeof(uint16_t) * T * H, hipMemcpyDeviceToHost));
  HIPOK(hipMemcpy(dst, (const int32_t*)plan.dev + s.o_dst_row, sizeof(int32_t) * T * K,
                  hipMemcpyDeviceToHost));
  /* every rank receives exactly S*K rows, each row at most once */
  int* per_rank = (int*)calloc(R, sizeof(int));
  char* seen = (char*)calloc((size_t)s.recv_rows, 1);
  for (int i = 0; i < T * K; ++i) {
    CHECK(dst[i] >= 0 && dst[i] < s.recv_rows, "dst_row[%d] = %d", i, dst[i]);
    CHECK(!seen[dst[i]], "row %d mapped twice", dst[i]);
    seen[dst[i]] = 1;
    per_rank[dst[i] / s.NvS]++;
  }
  for (int r = 0; r < R; ++r) CHECK(per_rank[r] == S * K, "rank %d holds %d", r, per_rank[r]);
  for (int i = 0; i < T * K; ++i) {
    HIPOK(hipMemcpy(row, (const uint16_t*)d_recv + (size_t)dst[i] * H, sizeof(uint16_t) * H,
                    hipMemcpyDeviceToHost));
    CHECK(memcmp(row, x + (size_t)(i / K) * H, sizeof(uint16_t) * H) == 0, "recv row of %d", i);
  }
  CHECK(memcmp(out, x, sizeof(uint16_t) * T * H) == 0, "combine of K equal rows, w = 1/K");
  HIPOK(hipStreamDestroy(st));
  hipFree(d_ids); hipFree(d_w); hipFree(d_plan); hipFree(d_ws);
  hipFree(d_x); hipFree(d_recv); hipFree(d_out);
  free(ids); free(w); free(x); free(out); free(dst); free(row); free(per_rank); free(seen);
  printf("gpu run ok: %d replicas, %d fallback pieces\n", stats.n_replicas, stats.n_fallback);
  return 0;
}

int main(int argc, char** argv) {
  if (argc < 2) return 2;
  if (strcmp(argv[1], "host") == 0) return host_checks();
  if (strcmp(argv[1], "gpu") == 0) return host_checks() || gpu_run();
  return 2;
}
