/* The C ABI used from plain C: one Reassign Cache step and one forward on a layer whose keys
 * and values are constant within each cluster (token j belongs to cluster j mod C, its key and
 * value are that cluster's rows). There the cluster representatives stand in exactly for the
 * keys they replace, so for any exact-block mask the output must be dense softmax attention,
 * which this program computes on the host in double precision and compares. It also checks
 * the assignment (every key to its own cluster), the sizes and the per-query-block counts
 * (keys of c outside b's exact blocks). fp32 plan, d = 64, B = 64, N = 300 (a ragged last
 * block), two heads, one shared mask with an empty row and a full row.
 * Prints "c abi ok" and exits 0 on success; prints the first mismatch and exits 1 otherwise. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "decoupattn.h"

#define H 2
#define N 300
#define D 64
#define B 64
#define C 8
#define NB ((N + B - 1) / B)

static uint32_t lcg_state = 12345u;
static float uniform(void) { /* in [-1, 1) */
  lcg_state = lcg_state * 1664525u + 1013904223u;
  return (float)((lcg_state >> 8) * (1.0 / 16777216.0)) * 2.f - 1.f;
}

#define CHECK_DA(call)                                                          \
  do {                                                                          \
    da_status st_ = (call);                                                     \
    if (st_ != DA_OK) {                                                         \
      printf("%s failed: %s\n", #call, da_status_str(st_));                     \
      return 1;                                                                 \
    }                                                                           \
  } while (0)
#define CHECK_HIP(call)                                                         \
  do {                                                                          \
    if ((call) != hipSuccess) {                                                 \
      printf("%s failed\n", #call);                                             \
      return 1;                                                                 \
    }                                                                           \
  } while (0)

int main(void) {
  static float Q[H][N][D], K[H][N][D], V[H][N][D], mu0[H][C][D], O[H][N][D];
  static float kc[H][C][D], vc[H][C][D];
  static int32_t assign[H][N], sizes[H][C], counts[H][NB][C];
  uint8_t mask[NB][NB];
  for (int h = 0; h < H; ++h)
    for (int c = 0; c < C; ++c)
      for (int i = 0; i < D; ++i) {
        kc[h][c][i] = uniform();
        vc[h][c][i] = uniform();
      }
  for (int h = 0; h < H; ++h)
    for (int j = 0; j < N; ++j)
      for (int i = 0; i < D; ++i) {
        Q[h][j][i] = uniform();
        K[h][j][i] = kc[h][j % C][i];
        V[h][j][i] = vc[h][j % C][i];
      }
  /* the cache starts a little off the cluster rows, so the refresh has work to do */
  for (int h = 0; h < H; ++h)
    for (int c = 0; c < C; ++c)
      for (int i = 0; i < D; ++i) mu0[h][c][i] = kc[h][c][i] + 0.01f * uniform();
  for (int b = 0; b < NB; ++b)
    for (int kb = 0; kb < NB; ++kb) mask[b][kb] = (uint8_t)(kb == b || (b + kb) % 3 == 0);
  for (int kb = 0; kb < NB; ++kb) {
    mask[1][kb] = 0;  /* query block 1: no exact block, compensation only */
    mask[3][kb] = 1;  /* query block 3: every block exact */
  }

  da_desc desc = {H, N, D, B, C, 1, DA_DTYPE_F32, 0.f, 0};
  da_plan plan = NULL;
  CHECK_DA(da_plan_create(&desc, &mask[0][0], &plan));

  void *dQ, *dK, *dV, *dmu0, *dmu1, *dvbar, *dO, *dassign, *dsizes, *dcounts;
  const size_t tok = sizeof(float) * H * N * D, cl = sizeof(float) * H * C * D;
  CHECK_HIP(hipMalloc(&dQ, tok));
  CHECK_HIP(hipMalloc(&dK, tok));
  CHECK_HIP(hipMalloc(&dV, tok));
  CHECK_HIP(hipMalloc(&dO, tok));
  CHECK_HIP(hipMalloc(&dmu0, cl));
  CHECK_HIP(hipMalloc(&dmu1, cl));
  CHECK_HIP(hipMalloc(&dvbar, cl));
  CHECK_HIP(hipMalloc(&dassign, sizeof(assign)));
  CHECK_HIP(hipMalloc(&dsizes, sizeof(sizes)));
  CHECK_HIP(hipMalloc(&dcounts, sizeof(counts)));
  CHECK_HIP(hipMemcpy(dQ, Q, tok, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dK, K, tok, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dV, V, tok, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dmu0, mu0, cl, hipMemcpyHostToDevice));

  CHECK_DA(da_reassign(plan, dK, dV, dmu0, dmu1, dvbar, (int32_t*)dassign, (int32_t*)dsizes,
                       (int32_t*)dcounts, NULL));
  CHECK_DA(da_forward(plan, dQ, dK, dV, dmu1, dvbar, (const int32_t*)dcounts, dO, NULL, NULL));
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(O, dO, tok, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(assign, dassign, sizeof(assign), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(sizes, dsizes, sizeof(sizes), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(counts, dcounts, sizeof(counts), hipMemcpyDeviceToHost));

  for (int h = 0; h < H; ++h) {
    for (int j = 0; j < N; ++j)
      if (assign[h][j] != j % C) {
        printf("head %d key %d assigned to %d, not %d\n", h, j, assign[h][j], j % C);
        return 1;
      }
    for (int c = 0; c < C; ++c)
      if (sizes[h][c] != N / C + (c < N % C)) {
        printf("head %d cluster %d size %d\n", h, c, sizes[h][c]);
        return 1;
      }
    for (int b = 0; b < NB; ++b)
      for (int c = 0; c < C; ++c) {
        int n = 0;
        for (int j = 0; j < N; ++j) n += (j % C == c) && !mask[b][j / B];
        if (counts[h][b][c] != n) {
          printf("head %d block %d cluster %d count %d, expected %d\n", h, b, c, counts[h][b][c], n);
          return 1;
        }
      }
  }
  /* dense attention on the host, double precision */
  const double scale = 1.0 / sqrt((double)D);
  static double s[N];
  double worst = 0.0;
  for (int h = 0; h < H; ++h)
    for (int i = 0; i < N; ++i) {
      double m = -INFINITY, tot = 0.0, o[D] = {0};
      for (int j = 0; j < N; ++j) {
        double dot = 0.0;
        for (int e = 0; e < D; ++e) dot += (double)Q[h][i][e] * K[h][j][e];
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
      }
      for (int j = 0; j < N; ++j) {
        const double w = exp(s[j] - m);
        tot += w;
        for (int e = 0; e < D; ++e) o[e] += w * V[h][j][e];
      }
      double num = 0.0, den = 0.0;
      for (int e = 0; e < D; ++e) {
        const double ref = o[e] / tot, diff = O[h][i][e] - ref;
        num += diff * diff;
        den += ref * ref;
      }
      const double rel = sqrt(num / (den + 1e-300));
      if (rel > worst) worst = rel;
    }
  CHECK_DA(da_plan_destroy(plan));
  hipFree(dQ); hipFree(dK); hipFree(dV); hipFree(dO); hipFree(dmu0); hipFree(dmu1);
  hipFree(dvbar); hipFree(dassign); hipFree(dsizes); hipFree(dcounts);
  if (!(worst <= 1e-5)) {
    printf("forward differs from dense attention: worst row relative L2 %.3g\n", worst);
    return 1;
  }
  printf("c abi ok (worst row relative L2 to dense attention %.2g)\n", worst);
  return 0;
}
