/*
 * host_cost.c -- host-side cost of the row-operator library's C ABI, timed
 * from plain C (no Python), as the launcher cost that the page "The TileLang
 * kernel DSL in DeepSeek-V4" (host code generation) puts under one
 * microsecond for its generated launchers.
 *
 *   host_cost validate [N]  argument validation alone: N calls that fail
 *                           validation (a NULL pointer) and N empty calls
 *                           (zero tokens) of rmsnorm_rope_fp8_fwd and of
 *                           rmsnorm_fwd.  Neither touches a device.
 *   host_cost launch [N]    N valid, asynchronous calls of
 *                           rmsnorm_rope_fp8_fwd (4096 tokens x 32 x 128,
 *                           bf16) on one stream, host time per call, then the
 *                           same for a bare launch of the same grid
 *                           (qrw_probe_empty).  Needs a GPU.
 *
 * Prints one "key value" line per figure (nanoseconds or microseconds per
 * call) and exits non-zero if a call returns an unexpected status.
 */
#define _POSIX_C_SOURCE 199309L
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#include <hip/hip_runtime_api.h>

#include "qrw.h"
#include "qrw_probe.h"

static double now_ns(void) {
  struct timespec ts;
  clock_gettime(CLOCK_MONOTONIC, &ts);
  return (double)ts.tv_sec * 1e9 + (double)ts.tv_nsec;
}

static int fails = 0;

static void expect(const char* what, int got, int want) {
  if (got != want) {
    fprintf(stderr, "%s: status %d (%s), want %d\n", what, got, qrw_status_string(got), want);
    ++fails;
  }
}

static int validate(int n) {
  void* x = (void*)(uintptr_t)(1ull << 32); /* never dereferenced */
  void* y = (void*)(uintptr_t)(2ull << 32);
  double t0 = now_ns();
  for (int i = 0; i < n; ++i)
    expect("fused null", rmsnorm_rope_fp8_fwd(NULL, x, x, x, (uint8_t*)y, (float*)y, 4096, 32, 128,
                                              128, 4096, 4096, QRW_BF16, QRW_BF16, 1, 1e-6f, NULL),
           QRW_ERR_NULL);
  double t1 = now_ns();
  for (int i = 0; i < n; ++i)
    expect("fused empty", rmsnorm_rope_fp8_fwd(x, x, x, x, (uint8_t*)y, (float*)y, 0, 32, 128, 128,
                                               4096, 4096, QRW_BF16, QRW_BF16, 1, 1e-6f, NULL),
           QRW_OK);
  double t2 = now_ns();
  for (int i = 0; i < n; ++i)
    expect("rmsnorm null", rmsnorm_fwd(NULL, x, y, 4096, 4096, 4096, 4096, QRW_F16, 1e-6f, NULL),
           QRW_ERR_NULL);
  double t3 = now_ns();
  for (int i = 0; i < n; ++i)
    expect("rmsnorm empty", rmsnorm_fwd(x, x, y, 0, 4096, 4096, 4096, QRW_F16, 1e-6f, NULL), QRW_OK);
  double t4 = now_ns();
  printf("calls %d\n", n);
  printf("fused_invalid_ns_per_call %.1f\n", (t1 - t0) / n);
  printf("fused_empty_ns_per_call %.1f\n", (t2 - t1) / n);
  printf("rmsnorm_invalid_ns_per_call %.1f\n", (t3 - t2) / n);
  printf("rmsnorm_empty_ns_per_call %.1f\n", (t4 - t3) / n);
  return fails ? 1 : 0;
}

#define HIP_OK(call)                                                         \
  do {                                                                       \
    hipError_t e_ = (call);                                                  \
    if (e_ != hipSuccess) {                                                  \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));             \
      return 2;                                                              \
    }                                                                        \
  } while (0)

static int launch(int n) {
  const int64_t T = 4096, N = 4096;
  void *x, *w, *c, *s, *q, *sc, *e;
  HIP_OK(hipMalloc(&x, T * N * 2));
  HIP_OK(hipMalloc(&w, N * 2));
  HIP_OK(hipMalloc(&c, T * 64 * 2));
  HIP_OK(hipMalloc(&s, T * 64 * 2));
  HIP_OK(hipMalloc(&q, T * N));
  HIP_OK(hipMalloc(&sc, T * 4));
  HIP_OK(hipMalloc(&e, T * 4));
  /* zero rows: valid inputs (codes 0, the floor scale) */
  HIP_OK(hipMemset(x, 0, T * N * 2));
  HIP_OK(hipMemset(w, 0, N * 2));
  HIP_OK(hipMemset(c, 0, T * 64 * 2));
  HIP_OK(hipMemset(s, 0, T * 64 * 2));
  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));
  for (int i = 0; i < 10; ++i)
    expect("warm-up", rmsnorm_rope_fp8_fwd(x, w, c, s, (uint8_t*)q, (float*)sc, T, 32, 128, 128, N,
                                           N, QRW_BF16, QRW_BF16, 1, 1e-6f, st),
           QRW_OK);
  HIP_OK(hipStreamSynchronize(st));
  double t0 = now_ns();
  for (int i = 0; i < n; ++i)
    expect("fused", rmsnorm_rope_fp8_fwd(x, w, c, s, (uint8_t*)q, (float*)sc, T, 32, 128, 128, N, N,
                                         QRW_BF16, QRW_BF16, 1, 1e-6f, st),
           QRW_OK);
  double t1 = now_ns();
  HIP_OK(hipStreamSynchronize(st));
  double t2 = now_ns();
  for (int i = 0; i < 10; ++i) expect("empty warm-up", qrw_probe_empty((uint32_t*)e, T / 4, st), QRW_OK);
  HIP_OK(hipStreamSynchronize(st));
  double t3 = now_ns();
  for (int i = 0; i < n; ++i) expect("empty", qrw_probe_empty((uint32_t*)e, T / 4, st), QRW_OK);
  double t4 = now_ns();
  HIP_OK(hipStreamSynchronize(st));
  double t5 = now_ns();
  printf("calls %d\n", n);
  printf("fused_launch_host_us_per_call %.3f\n", (t1 - t0) / n * 1e-3);
  printf("fused_calls_plus_sync_us_per_call %.3f\n", (t2 - t0) / n * 1e-3);
  printf("bare_launch_host_us_per_call %.3f\n", (t4 - t3) / n * 1e-3);
  printf("bare_calls_plus_sync_us_per_call %.3f\n", (t5 - t3) / n * 1e-3);
  HIP_OK(hipStreamDestroy(st));
  hipFree(x);
  hipFree(w);
  hipFree(c);
  hipFree(s);
  hipFree(q);
  hipFree(sc);
  hipFree(e);
  return fails ? 1 : 0;
}

int main(int argc, char** argv) {
  const char* mode = argc > 1 ? argv[1] : "validate";
  int n = argc > 2 ? atoi(argv[2]) : 0;
  if (strcmp(mode, "validate") == 0) return validate(n > 0 ? n : 1000000);
  if (strcmp(mode, "launch") == 0) return launch(n > 0 ? n : 200);
  fprintf(stderr, "usage: host_cost validate|launch [N]\n");
  return 2;
}
