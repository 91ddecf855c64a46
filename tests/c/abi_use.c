/* The C ABI used from C alone, with no Python or torch: device buffers from
 * hipMalloc, a 16-rank ring all-reduce, then a reduce-scatter and an
 * all-gather through ar.h, each checked on the host against exact sums.
 * The inputs are small integers, so every partial sum is exact in fp32 and
 * the result does not depend on the order of the adds.  Prints "ok" and
 * returns 0 on success; prints what failed and returns 1 otherwise. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "ar.h"

#define N 16
#define COUNT ((size_t)(1 << 20) + 37)

static int fail(const char *what) {
  printf("FAIL: %s (%s)\n", what, ar_last_error());
  return 1;
}

static float input(int r, size_t e) { return (float)((int)((e * 7 + (size_t)r * 13) % 11) - 5); }

static float sum(size_t e) {
  float s = 0.0f;
  for (int r = 0; r < N; ++r) s += input(r, e);
  return s;
}

static int upload(void *const *d, float *h) {
  for (int r = 0; r < N; ++r) {
    for (size_t e = 0; e < COUNT; ++e) h[e] = input(r, e);
    if (hipMemcpy(d[r], h, COUNT * sizeof(float), hipMemcpyHostToDevice) != hipSuccess) return 1;
  }
  return 0;
}

int main(void) {
  void *d[N];
  float *h = (float *)malloc(COUNT * sizeof(float));
  if (!h) return fail("host allocation");
  for (int r = 0; r < N; ++r)
    if (hipMalloc(&d[r], COUNT * sizeof(float)) != hipSuccess) return fail("hipMalloc");

  /* the all-reduce: every rank ends with the sum */
  if (upload(d, h)) return fail("upload");
  ar_plan_t *p = ar_plan_create(N, 8, COUNT, AR_FLOAT32, AR_RING);
  if (!p) return fail("ar_plan_create");
  if (ar_allreduce(p, d, NULL) != AR_OK) return fail("ar_allreduce");
  if (hipDeviceSynchronize() != hipSuccess) return fail("hipDeviceSynchronize");
  ar_stats_t st = ar_plan_stats(p);
  if (st.steps != 2 * (N - 1)) return fail("ring steps");
  for (int r = 0; r < N; ++r) {
    if (hipMemcpy(h, d[r], COUNT * sizeof(float), hipMemcpyDeviceToHost) != hipSuccess) return fail("download");
    for (size_t e = 0; e < COUNT; ++e)
      if (h[e] != sum(e)) return fail("all-reduce value");
  }
  ar_plan_destroy(p);

  /* the two halves, one-pass: the owned ranges after the reduce-scatter,
     everything after the all-gather */
  if (upload(d, h)) return fail("upload");
  ar_plan_t *rs = ar_plan_create_collective(N, 8, COUNT, AR_FLOAT32, AR_RING, AR_REDUCE_SCATTER);
  ar_plan_t *ag = ar_plan_create_collective(N, 8, COUNT, AR_FLOAT32, AR_RING, AR_ALLGATHER);
  if (!rs || !ag) return fail("ar_plan_create_collective");
  if (ar_plan_set_exec(rs, AR_EXEC_ONEPASS) != AR_OK || ar_plan_set_exec(ag, AR_EXEC_ONEPASS) != AR_OK)
    return fail("ar_plan_set_exec");
  if (ar_reduce_scatter(rs, d, NULL) != AR_OK) return fail("ar_reduce_scatter");
  if (hipDeviceSynchronize() != hipSuccess) return fail("hipDeviceSynchronize");
  size_t covered = 0;
  for (int r = 0; r < N; ++r) {
    size_t lo = 0, hi = 0;
    if (ar_plan_owned_range(rs, r, &lo, &hi) != AR_OK) return fail("ar_plan_owned_range");
    covered += hi - lo;
    if (hipMemcpy(h, d[r], COUNT * sizeof(float), hipMemcpyDeviceToHost) != hipSuccess) return fail("download");
    for (size_t e = 0; e < COUNT; ++e) {
      const float want = (e >= lo && e < hi) ? sum(e) : input(r, e);
      if (h[e] != want) return fail("reduce-scatter value");
    }
  }
  if (covered != COUNT) return fail("owned ranges do not cover the buffer");
  if (ar_allgather(ag, d, NULL) != AR_OK) return fail("ar_allgather");
  if (hipDeviceSynchronize() != hipSuccess) return fail("hipDeviceSynchronize");
  for (int r = 0; r < N; ++r) {
    if (hipMemcpy(h, d[r], COUNT * sizeof(float), hipMemcpyDeviceToHost) != hipSuccess) return fail("download");
    for (size_t e = 0; e < COUNT; ++e)
      if (h[e] != sum(e)) return fail("all-gather value");
  }
  /* a plan runs only through its own collective's call */
  if (ar_allreduce(rs, d, NULL) != AR_ERR_INVALID_ARG) return fail("ar_allreduce accepted a reduce-scatter plan");
  ar_plan_destroy(rs);
  ar_plan_destroy(ag);
  for (int r = 0; r < N; ++r) hipFree(d[r]);
  free(h);
  printf("ok\n");
  return 0;
}
