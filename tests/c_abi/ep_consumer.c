/*
 * A plain C99 user of the library: include/ep.h compiled by a C compiler,
 * libep.so linked, no Python and no C++.
 *
 *   ep_consumer host   host-only calls (size queries, argument checks that
 *                      fail before any launch, the last-error text); needs
 *                      no GPU
 *   ep_consumer gpu    one layout -> dispatch -> combine round trip on the
 *                      current GPU, checked against the closed form of the
 *                      "Low-Latency Mode API" pair: with bf16 rows (no
 *                      quantisation) as the expert outputs and unit weights,
 *                      combine returns k_eff * x for every token, exactly
 *                      (k_eff <= 4 equal terms of a bf16 value sum exactly in
 *                      float32 and round back to bf16 without loss for the
 *                      small integers used here)
 *
 * Prints one line per check and exits non-zero on the first failure.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "ep.h"

static int fails = 0;

static void check(int ok, const char *what) {
  printf("%s %s\n", ok ? "ok  " : "FAIL", what);
  if (!ok) ++fails;
}

static int host_checks(void) {
  check(ep_abi_version() == EP_ABI_VERSION, "ep_abi_version matches the header");
  check(ep_workspace_bytes(128, 8, 256) > 0, "ep_workspace_bytes of a decode shape");
  check(ep_workspace_bytes(128, 0, 256) == 0, "ep_workspace_bytes rejects k = 0");
  check(ep_layout_rows(128, 8, 256, 1, 0) == 1024, "compact rows = T_max * k");
  check(ep_layout_rows(128, 8, 256, 1, 16) == 256 * 16, "capacity rows = E * C");

  size_t total = 0, scale_off = 0;
  check(ep_buffer_bytes(1024, 7168, EP_QUANT_MXFP8, &total, &scale_off) == EP_OK, "ep_buffer_bytes MXFP8");
  check(scale_off == (size_t)1024 * 7168 && total == scale_off + (size_t)1024 * 224,
        "MXFP8 data region, then 224 scale bytes per row");
  check(ep_buffer_bytes(16, 100, EP_QUANT_MXFP8, &total, &scale_off) == EP_ERR_INVALID_ARG,
        "ep_buffer_bytes rejects H % 32 != 0");

  /* a layout call with a NULL workspace fails on the host and says why */
  ep_handle_t h;
  const ep_status_t st = ep_layout((const void *)0x1000, EP_IDX_INT64, 4, 2, 4, 8, (int64_t *)0x1000, NULL, NULL,
                                   0, &h, NULL);
  check(st == EP_ERR_INVALID_ARG, "ep_layout rejects a NULL workspace before launching");
  check(strlen(ep_last_error()) > 0, "ep_last_error describes the failed check");
  return fails;
}

static uint16_t bf16_of_small_int(int v) {
  /* v in [-8, 8]: exact in bf16 (8 significant bits) */
  float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

#define HIPCHECK(x)                                                  \
  do {                                                               \
    hipError_t e_ = (x);                                             \
    if (e_ != hipSuccess) {                                          \
      printf("FAIL %s: %s\n", #x, hipGetErrorString(e_));            \
      return 1;                                                      \
    }                                                                \
  } while (0)

static int gpu_round_trip(void) {
  enum { T = 6, K = 4, E = 8, H = 256 };
  int64_t idx[T * K];
  float wts[T * K];
  uint16_t x[T * H];
  int keff[T];
  /* token t: experts (t + 3j) % E for j < K, with some slots unrouted */
  for (int t = 0; t < T; ++t) {
    keff[t] = 0;
    for (int j = 0; j < K; ++j) {
      const int unrouted = (t == 1 && j == 2) || (t == 4) || (t == 5 && j == 0);
      idx[t * K + j] = unrouted ? -1 : (t + 3 * j) % E;
      keff[t] += !unrouted;
      wts[t * K + j] = 1.0f;
    }
    for (int c = 0; c < H; ++c) x[t * H + c] = bf16_of_small_int((t * 7 + c) % 5 - 2);
  }

  const size_t ws_bytes = ep_workspace_bytes(T, K, E);
  const int64_t rows = ep_layout_rows(T, K, E, 1, 0);
  size_t buf_bytes = 0;
  if (ws_bytes == 0 || rows <= 0 || ep_buffer_bytes(rows, H, EP_QUANT_NONE, &buf_bytes, NULL) != EP_OK) {
    printf("FAIL size queries\n");
    return 1;
  }
  void *d_idx, *d_wts, *d_x, *d_ws, *d_recv, *d_out, *d_cnt;
  HIPCHECK(hipMalloc(&d_idx, sizeof idx));
  HIPCHECK(hipMalloc(&d_wts, sizeof wts));
  HIPCHECK(hipMalloc(&d_x, sizeof x));
  HIPCHECK(hipMalloc(&d_ws, ws_bytes));
  HIPCHECK(hipMalloc(&d_recv, buf_bytes));
  HIPCHECK(hipMalloc(&d_out, sizeof x));
  HIPCHECK(hipMalloc(&d_cnt, E * sizeof(int64_t)));
  HIPCHECK(hipMemcpy(d_idx, idx, sizeof idx, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(d_wts, wts, sizeof wts, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(d_x, x, sizeof x, hipMemcpyHostToDevice));

  ep_handle_t h;
  check(ep_layout(d_idx, EP_IDX_INT64, T, K, T, E, (int64_t *)d_cnt, NULL, d_ws, ws_bytes, &h, NULL) == EP_OK,
        "ep_layout");
  check(ep_dispatch(&h, d_x, H, NULL, EP_QUANT_NONE, d_recv, buf_bytes, NULL, NULL) == EP_OK, "ep_dispatch");
  check(ep_combine(&h, d_recv, buf_bytes, EP_QUANT_NONE, H, d_idx, EP_IDX_INT64, (const float *)d_wts, d_out,
                   NULL) == EP_OK,
        "ep_combine");
  uint32_t flags = 99;
  check(ep_read_status(&h, &flags, NULL) == EP_OK && flags == 0, "status word clear");

  uint16_t out[T * H];
  int64_t cnt[E];
  HIPCHECK(hipMemcpy(out, d_out, sizeof out, hipMemcpyDeviceToHost));
  HIPCHECK(hipMemcpy(cnt, d_cnt, sizeof cnt, hipMemcpyDeviceToHost));

  int64_t want_cnt[E] = {0}, routed = 0, got = 0;
  for (int f = 0; f < T * K; ++f)
    if (idx[f] >= 0) ++want_cnt[idx[f]], ++routed;
  int cnt_ok = 1;
  for (int e = 0; e < E; ++e) cnt_ok &= cnt[e] == want_cnt[e], got += cnt[e];
  check(cnt_ok && got == routed, "recv_count is the expert histogram");

  int out_ok = 1;
  for (int t = 0; t < T; ++t)
    for (int c = 0; c < H; ++c) {
      const int v = (t * 7 + c) % 5 - 2;
      const uint16_t want = keff[t] ? bf16_of_small_int(keff[t] * v) : 0; /* +0 for a token routed nowhere */
      out_ok &= out[t * H + c] == want;
    }
  check(out_ok, "combine(dispatch(x)) == k_eff * x for every token");

  hipFree(d_idx);
  hipFree(d_wts);
  hipFree(d_x);
  hipFree(d_ws);
  hipFree(d_recv);
  hipFree(d_out);
  hipFree(d_cnt);
  return fails;
}

int main(int argc, char **argv) {
  if (argc != 2 || (strcmp(argv[1], "host") != 0 && strcmp(argv[1], "gpu") != 0)) {
    fprintf(stderr, "usage: %s host|gpu\n", argv[0]);
    return 2;
  }
  const int r = strcmp(argv[1], "host") == 0 ? host_checks() : gpu_round_trip();
  printf("%s\n", r == 0 ? "all checks passed" : "some checks failed");
  return r == 0 ? 0 : 1;
}
