/*
 * oracle_driver.c — calls every function of the fp64 oracle (oracle/
 * mita_oracle.h) on small seeded inputs, including its edge cases (k == N,
 * m == 1, m == N, query subsets, s > 1, ragged windows), so that a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer (tests/
 * test_oracle_sanitize.py) sees every loop of it run.  It checks only a few
 * return codes and shapes: the values are pinned elsewhere.
 * Test infrastructure only.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "mita_oracle.h"

static uint64_t state = 0x9E3779B97F4A7C15ull;

static double next_normal(void) { /* Box-Muller on a 64-bit LCG: data only */
  state = state * 6364136223846793005ull + 1442695040888963407ull;
  double u1 = ((state >> 11) + 1.0) / 9007199254740993.0;
  state = state * 6364136223846793005ull + 1442695040888963407ull;
  double u2 = (state >> 11) / 9007199254740992.0;
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

static double* randn(int64_t n) {
  double* p = (double*)malloc((size_t)n * sizeof(double));
  for (int64_t i = 0; i < n; ++i) p[i] = next_normal();
  return p;
}

#define CHECK(x)                                                   \
  do {                                                             \
    int rc_ = (x);                                                 \
    if (rc_ != 0) {                                                \
      fprintf(stderr, "%s:%d: %s returned %d\n", __FILE__, __LINE__, #x, rc_); \
      return 1;                                                    \
    }                                                              \
  } while (0)

static int one_case(int64_t N, int64_t d, int64_t gh, int64_t gw, int64_t mh, int64_t mw,
                    int64_t k, int round_mode) {
  const int64_t m = mh * mw;
  double* Q = randn(N * d);
  double* K = randn(N * d);
  double* V = randn(N * d);
  double* Ql = (double*)malloc((size_t)(m * d) * sizeof(double));
  double* Vl = (double*)malloc((size_t)(m * d) * sizeof(double));
  int32_t* idx = (int32_t*)malloc((size_t)(m * k) * sizeof(int32_t));
  double* gap = (double*)malloc((size_t)(m * 4) * sizeof(double));
  int32_t* route = (int32_t*)malloc((size_t)N * sizeof(int32_t));
  double* top2 = (double*)malloc((size_t)(N * 4) * sizeof(double));
  int32_t* offsets = (int32_t*)malloc((size_t)(m + 1) * sizeof(int32_t));
  int32_t* perm = (int32_t*)malloc((size_t)N * sizeof(int32_t));
  double* out = (double*)malloc((size_t)(N * d) * sizeof(double));
  int64_t qsel[3] = {0, N / 2, N - 1};

  for (int64_t i = 0; i < m; ++i) {
    int64_t r0, r1, c0, c1;
    CHECK(mita_oracle_window(gh, gw, mh, mw, i, &r0, &r1, &c0, &c1));
  }
  CHECK(mita_oracle_pool(Q, N, d, gh, gw, mh, mw, round_mode, Ql));
  CHECK(mita_oracle_topk(Ql, K, N, d, m, k, idx, gap));
  CHECK(mita_oracle_topk(Ql, K, N, d, m, k, idx, NULL));
  CHECK(mita_oracle_landmark_values(Ql, K, V, N, d, m, 0.125, Vl));
  CHECK(mita_oracle_route(Q, Ql, N, d, m, NULL, N, route, top2));
  CHECK(mita_oracle_route(Q, Ql, N, d, m, qsel, 3, route, top2));
  CHECK(mita_oracle_route(Q, Ql, N, d, m, NULL, N, route, NULL));
  CHECK(mita_oracle_bucket(route, N, m, offsets, perm));
  CHECK(mita_oracle_output(Q, K, V, Ql, Vl, idx, route, N, d, m, k, 0.125, NULL, N, out));
  CHECK(mita_oracle_output(Q, K, V, Ql, Vl, idx, route, N, d, m, k, 0.125, qsel, 3, out));
  CHECK(mita_oracle_dense(Q, K, V, N, d, 0.125, NULL, N, out));
  CHECK(mita_oracle_dense(Q, K, V, N, d, 0.125, qsel, 3, out));

  /* two slices through the composed forward, every optional output */
  double* Q2 = randn(2 * N * d);
  double* K2 = randn(2 * N * d);
  double* V2 = randn(2 * N * d);
  double* out2 = (double*)malloc((size_t)(2 * N * d) * sizeof(double));
  int32_t* idx2 = (int32_t*)malloc((size_t)(2 * m * k) * sizeof(int32_t));
  int32_t* route2 = (int32_t*)malloc((size_t)(2 * N) * sizeof(int32_t));
  double* Ql2 = (double*)malloc((size_t)(2 * m * d) * sizeof(double));
  double* Vl2 = (double*)malloc((size_t)(2 * m * d) * sizeof(double));
  int32_t* off2 = (int32_t*)malloc((size_t)(2 * (m + 1)) * sizeof(int32_t));
  int32_t* perm2 = (int32_t*)malloc((size_t)(2 * N) * sizeof(int32_t));
  CHECK(mita_oracle_forward(Q2, K2, V2, 1, 2, N, d, gh, gw, mh, mw, k, 0.125, round_mode, out2,
                            idx2, route2, Ql2, Vl2, off2, perm2));
  CHECK(mita_oracle_forward(Q2, K2, V2, 2, 1, N, d, gh, gw, mh, mw, k, 0.125, round_mode, out2,
                            idx2, route2, NULL, NULL, NULL, NULL));

  /* several experts per query */
  for (int64_t s = 1; s <= (m < 3 ? m : 3); ++s) {
    int32_t* rs = (int32_t*)malloc((size_t)(N * s) * sizeof(int32_t));
    int32_t* offs = (int32_t*)malloc((size_t)(m + 1) * sizeof(int32_t));
    int32_t* perms = (int32_t*)malloc((size_t)(N * s) * sizeof(int32_t));
    CHECK(mita_oracle_route_s(Q, Ql, N, d, m, s, NULL, N, rs));
    CHECK(mita_oracle_bucket_s(rs, N, m, s, offs, perms));
    CHECK(mita_oracle_output_s(Q, K, V, Ql, Vl, idx, rs, N, d, m, k, s, 0.125, NULL, N, out));
    CHECK(mita_oracle_output_s(Q, K, V, Ql, Vl, idx, rs, N, d, m, k, s, 0.125, qsel, 3, out));
    free(rs);
    free(offs);
    free(perms);
  }
  /* the backward pass with these experts and routes */
  {
    double* G = randn(N * d);
    double* dQ = (double*)malloc((size_t)(N * d) * sizeof(double));
    double* dK = (double*)malloc((size_t)(N * d) * sizeof(double));
    double* dV = (double*)malloc((size_t)(N * d) * sizeof(double));
    CHECK(mita_oracle_backward(Q, K, V, N, d, gh, gw, mh, mw, k, 0.125, round_mode, idx, route,
                               G, dQ, dK, dV));
    free(G);
    free(dQ);
    free(dK);
    free(dV);
  }
  (void)mita_oracle_round_bf16(3.14159);
  (void)mita_oracle_round_bf16(-1e-40);
  (void)mita_oracle_round_bf16(1e39);

  free(Q); free(K); free(V); free(Ql); free(Vl); free(idx); free(gap); free(route);
  free(top2); free(offsets); free(perm); free(out);
  free(Q2); free(K2); free(V2); free(out2); free(idx2); free(route2); free(Ql2); free(Vl2);
  free(off2); free(perm2);
  return 0;
}

int main(void) {
  /* 14x14 grid to 5x5 (overlapping bins), bf16 rounding */
  if (one_case(196, 16, 14, 14, 5, 5, 25, MITA_ORACLE_ROUND_BF16)) return 1;
  /* ragged 1D windows, k == N, fp32 rounding */
  if (one_case(37, 8, 1, 37, 1, 5, 37, MITA_ORACLE_ROUND_F32)) return 1;
  /* one landmark, k == 1 */
  if (one_case(50, 4, 1, 50, 1, 1, 1, MITA_ORACLE_ROUND_NONE)) return 1;
  /* m == N (every window one token) */
  if (one_case(16, 4, 4, 4, 4, 4, 3, MITA_ORACLE_ROUND_BF16)) return 1;
  /* argument errors are reported, not acted on */
  if (mita_oracle_topk(NULL, NULL, 0, 0, 0, 0, NULL, NULL) == 0) return 1;
  if (mita_oracle_pool(NULL, 1, 1, 1, 1, 2, 1, 0, NULL) == 0) return 1;
  if (mita_oracle_backward(NULL, NULL, NULL, 1, 1, 1, 1, 1, 1, 1, 1.0, 0, NULL, NULL, NULL, NULL,
                           NULL, NULL) == 0)
    return 1;
  printf("oracle sanitize driver: ok (%d threads)\n", mita_oracle_threads());
  return 0;
}
