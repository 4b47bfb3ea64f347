/*
 * mita_oracle.c — plain fp64 CPU oracle for the MiTA forward pass.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and the
 * benchmark's CPU-baseline leg; never by the GPU library.  See mita_oracle.h
 * for the page citations of each step.  Everything here is written for
 * readability: straight loops, fp64 throughout, full sorts where a sort
 * defines the result.  OpenMP only splits independent rows across threads;
 * every sum runs in a fixed sequential order.
 */
#include "mita_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int mita_oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Rounding into the input precision                                        */
/* ------------------------------------------------------------------------ */

double mita_oracle_round_bf16(double x) {
  if (isnan(x) || isinf(x) || x == 0.0) return x;
  int e;
  (void)frexp(x, &e); /* |x| in [2^(e-1), 2^e) */
  /* bfloat16 keeps 8 significant bits, so the spacing of representable
   * values around x is 2^(e-8); below the smallest normal (2^-126) the
   * spacing stays at the subnormal quantum 2^-133. */
  int q = e - 8;
  if (q < -133) q = -133;
  double r = ldexp(nearbyint(ldexp(x, -q)), q); /* nearbyint: ties to even */
  const double max_bf16 = ldexp(255.0, 120);      /* (2 - 2^-7) * 2^127 */
  if (fabs(r) > max_bf16) return copysign(INFINITY, x);
  return r;
}

static double round_to(double x, int mode) {
  switch (mode) {
    case MITA_ORACLE_ROUND_F32: {
      if (fabs(x) > 3.4028234663852886e38) {
        /* beyond the largest float: round-to-nearest goes to infinity only
         * past the midpoint to 2^128 */
        double mid = ldexp(1.0, 128) - ldexp(1.0, 103);
        if (fabs(x) >= mid) return copysign(INFINITY, x);
        return copysign(3.4028234663852886e38, x);
      }
      return (double)(float)x;
    }
    case MITA_ORACLE_ROUND_BF16:
      return mita_oracle_round_bf16(x);
    default:
      return x;
  }
}

/* ------------------------------------------------------------------------ */
/* Step 1: landmark queries by local average pooling                        */
/* ------------------------------------------------------------------------ */

static int64_t floor_div(int64_t a, int64_t b) { return a / b; }            /* a, b >= 0 */
static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; } /* a >= 0, b > 0 */

int mita_oracle_window(int64_t gh, int64_t gw, int64_t mh, int64_t mw, int64_t i,
                       int64_t* r0, int64_t* r1, int64_t* c0, int64_t* c1) {
  if (gh < 1 || gw < 1 || mh < 1 || mw < 1 || mh > gh || mw > gw) return -1;
  if (i < 0 || i >= mh * mw) return -1;
  int64_t a = i / mw, c = i % mw;
  *r0 = floor_div(a * gh, mh);
  *r1 = ceil_div((a + 1) * gh, mh);
  *c0 = floor_div(c * gw, mw);
  *c1 = ceil_div((c + 1) * gw, mw);
  return 0;
}

int mita_oracle_pool(const double* Q, int64_t N, int64_t d, int64_t gh, int64_t gw,
                     int64_t mh, int64_t mw, int round_mode, double* Ql) {
  if (!Q || !Ql || N < 1 || d < 1 || gh * gw != N) return -1;
  if (mh < 1 || mw < 1 || mh > gh || mw > gw) return -1;
  if (round_mode < 0 || round_mode > 2) return -1;
  const int64_t m = mh * mw;
  int bad = 0;
#pragma omp parallel for schedule(dynamic)
  for (int64_t i = 0; i < m; ++i) {
    int64_t r0, r1, c0, c1;
    if (mita_oracle_window(gh, gw, mh, mw, i, &r0, &r1, &c0, &c1) != 0) {
#pragma omp atomic write
      bad = 1;
      continue;
    }
    const double count = (double)((r1 - r0) * (c1 - c0));
    for (int64_t j = 0; j < d; ++j) {
      double sum = 0.0;
      for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = c0; c < c1; ++c) sum += Q[(r * gw + c) * d + j];
      Ql[i * d + j] = round_to(sum / count, round_mode);
    }
  }
  return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Step 2a: routed experts = per-landmark top-k keys                         */
/* ------------------------------------------------------------------------ */

static double dot(const double* a, const double* b, int64_t d) {
  double s = 0.0;
  for (int64_t j = 0; j < d; ++j) s += a[j] * b[j];
  return s;
}

static double abs_dot(const double* a, const double* b, int64_t d) {
  double s = 0.0;
  for (int64_t j = 0; j < d; ++j) s += fabs(a[j] * b[j]);
  return s;
}

typedef struct {
  double s;
  int64_t t;
} scored_t;

/* better-first: larger score, then lower index */
static int cmp_scored(const void* pa, const void* pb) {
  const scored_t* a = (const scored_t*)pa;
  const scored_t* b = (const scored_t*)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->t < b->t) ? -1 : (a->t > b->t);
}

static int cmp_i32(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a > b) - (a < b);
}

int mita_oracle_topk(const double* Ql, const double* K, int64_t N, int64_t d, int64_t m,
                     int64_t k, int32_t* idx, double* gap) {
  if (!Ql || !K || !idx || N < 1 || d < 1 || m < 1 || k < 1 || k > N) return -1;
  if (N > INT32_MAX) return -1;
  int fail = 0;
#pragma omp parallel
  {
    scored_t* row = (scored_t*)malloc((size_t)N * sizeof(scored_t));
    if (!row) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(dynamic)
    for (int64_t i = 0; i < m; ++i) {
      if (!row) continue;
      for (int64_t t = 0; t < N; ++t) {
        row[t].s = dot(Ql + i * d, K + t * d, d);
        row[t].t = t;
      }
      qsort(row, (size_t)N, sizeof(scored_t), cmp_scored);
      int32_t* dst = idx + i * k;
      for (int64_t j = 0; j < k; ++j) dst[j] = (int32_t)row[j].t;
      qsort(dst, (size_t)k, sizeof(int32_t), cmp_i32);
      if (gap) {
        double* g = gap + i * 4;
        g[0] = row[k - 1].s;
        g[2] = abs_dot(Ql + i * d, K + row[k - 1].t * d, d);
        if (k < N) {
          g[1] = row[k].s;
          g[3] = abs_dot(Ql + i * d, K + row[k].t * d, d);
        } else {
          g[1] = -INFINITY;
          g[3] = 0.0;
        }
      }
    }
    free(row);
  }
  return fail ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* Step 2b: landmark values = cross-attention of the landmarks over all keys */
/* ------------------------------------------------------------------------ */

int mita_oracle_landmark_values(const double* Ql, const double* K, const double* V,
                                int64_t N, int64_t d, int64_t m, double scale, double* Vl) {
  if (!Ql || !K || !V || !Vl || N < 1 || d < 1 || m < 1) return -1;
  if (!(scale > 0.0) || isinf(scale)) return -1;
  int fail = 0;
#pragma omp parallel
  {
    double* logit = (double*)malloc((size_t)N * sizeof(double));
    if (!logit) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(dynamic)
    for (int64_t i = 0; i < m; ++i) {
      if (!logit) continue;
      double mx = -INFINITY;
      for (int64_t t = 0; t < N; ++t) {
        logit[t] = scale * dot(Ql + i * d, K + t * d, d);
        if (logit[t] > mx) mx = logit[t];
      }
      double z = 0.0;
      for (int64_t t = 0; t < N; ++t) {
        logit[t] = exp(logit[t] - mx); /* now the unnormalised weight */
        z += logit[t];
      }
      for (int64_t j = 0; j < d; ++j) {
        double acc = 0.0;
        for (int64_t t = 0; t < N; ++t) acc += logit[t] * V[t * d + j];
        Vl[i * d + j] = acc / z;
      }
    }
    free(logit);
  }
  return fail ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* Step 3: routing, one expert per query                                    */
/* ------------------------------------------------------------------------ */

int mita_oracle_route(const double* Q, const double* Ql, int64_t N, int64_t d, int64_t m,
                      const int64_t* qsel, int64_t nq, int32_t* route, double* top2) {
  if (!Q || !Ql || !route || N < 1 || d < 1 || m < 1) return -1;
  if (!qsel && nq != N) return -1;
  if (nq < 0) return -1;
  int bad = 0;
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < nq; ++p) {
    const int64_t q = qsel ? qsel[p] : p;
    if (q < 0 || q >= N) {
#pragma omp atomic write
      bad = 1;
      continue;
    }
    int64_t best = 0;
    double best_v = dot(Q + q * d, Ql, d);
    for (int64_t i = 1; i < m; ++i) {
      double v = dot(Q + q * d, Ql + i * d, d);
      if (v > best_v) { /* strict: the first maximum is kept */
        best_v = v;
        best = i;
      }
    }
    route[p] = (int32_t)best;
    if (top2) {
      double second = -INFINITY;
      int64_t second_i = -1;
      for (int64_t i = 0; i < m; ++i) {
        if (i == best) continue;
        double v = dot(Q + q * d, Ql + i * d, d);
        if (v > second) {
          second = v;
          second_i = i;
        }
      }
      double* g = top2 + p * 4;
      g[0] = best_v;
      g[1] = second;
      g[2] = abs_dot(Q + q * d, Ql + best * d, d);
      g[3] = second_i >= 0 ? abs_dot(Q + q * d, Ql + second_i * d, d) : 0.0;
    }
  }
  return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Step 4: grouping queries by expert                                        */
/* ------------------------------------------------------------------------ */

int mita_oracle_bucket(const int32_t* route, int64_t N, int64_t m, int32_t* offsets,
                       int32_t* perm) {
  if (!route || !offsets || !perm || N < 1 || m < 1) return -1;
  for (int64_t e = 0; e <= m; ++e) offsets[e] = 0;
  for (int64_t q = 0; q < N; ++q) {
    if (route[q] < 0 || route[q] >= m) return -1;
    offsets[route[q] + 1] += 1;
  }
  for (int64_t e = 0; e < m; ++e) offsets[e + 1] += offsets[e];
  int32_t* fill = (int32_t*)malloc((size_t)m * sizeof(int32_t));
  if (!fill) return -2;
  for (int64_t e = 0; e < m; ++e) fill[e] = offsets[e];
  /* visiting queries in increasing index keeps each group in index order */
  for (int64_t q = 0; q < N; ++q) perm[fill[route[q]]++] = (int32_t)q;
  free(fill);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Step 5: query-expert attention over m compressed + k raw pairs            */
/* ------------------------------------------------------------------------ */

int mita_oracle_output(const double* Q, const double* K, const double* V, const double* Ql,
                       const double* Vl, const int32_t* idx, const int32_t* route, int64_t N,
                       int64_t d, int64_t m, int64_t k, double scale, const int64_t* qsel,
                       int64_t nq, double* out) {
  if (!Q || !K || !V || !Ql || !Vl || !idx || !route || !out) return -1;
  if (N < 1 || d < 1 || m < 1 || k < 1 || k > N) return -1;
  if (!(scale > 0.0) || isinf(scale)) return -1;
  if (!qsel && nq != N) return -1;
  if (nq < 0) return -1;
  int bad = 0;
#pragma omp parallel
  {
    double* w = (double*)malloc((size_t)(m + k) * sizeof(double));
    if (!w) {
#pragma omp atomic write
      bad = 2;
    }
#pragma omp for schedule(static)
    for (int64_t p = 0; p < nq; ++p) {
      if (!w) continue;
      const int64_t q = qsel ? qsel[p] : p;
      if (q < 0 || q >= N || route[q] < 0 || route[q] >= m) {
#pragma omp atomic write
        bad = 1;
        continue;
      }
      const int32_t* ex = idx + (int64_t)route[q] * k;
      /* logits: the m compressed keys first, then the expert's k raw keys */
      double mx = -INFINITY;
      for (int64_t i = 0; i < m; ++i) {
        w[i] = scale * dot(Q + q * d, Ql + i * d, d);
        if (w[i] > mx) mx = w[i];
      }
      for (int64_t j = 0; j < k; ++j) {
        w[m + j] = scale * dot(Q + q * d, K + (int64_t)ex[j] * d, d);
        if (w[m + j] > mx) mx = w[m + j];
      }
      double z = 0.0;
      for (int64_t i = 0; i < m + k; ++i) {
        w[i] = exp(w[i] - mx);
        z += w[i];
      }
      for (int64_t c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int64_t i = 0; i < m; ++i) acc += w[i] * Vl[i * d + c];
        for (int64_t j = 0; j < k; ++j) acc += w[m + j] * V[(int64_t)ex[j] * d + c];
        out[p * d + c] = acc / z;
      }
    }
    free(w);
  }
  return bad == 2 ? -2 : (bad ? -1 : 0);
}

/* ------------------------------------------------------------------------ */
/* Steps 3-5 with s experts per query (reading in mita_oracle.h)             */
/* ------------------------------------------------------------------------ */

int mita_oracle_route_s(const double* Q, const double* Ql, int64_t N, int64_t d, int64_t m,
                        int64_t s, const int64_t* qsel, int64_t nq, int32_t* routes) {
  if (!Q || !Ql || !routes || N < 1 || d < 1 || m < 1 || s < 1 || s > m) return -1;
  if (!qsel && nq != N) return -1;
  if (nq < 0) return -1;
  int bad = 0;
#pragma omp parallel
  {
    double* R = (double*)malloc((size_t)m * sizeof(double));
    char* taken = (char*)malloc((size_t)m);
    if (!R || !taken) {
#pragma omp atomic write
      bad = 2;
    }
#pragma omp for schedule(static)
    for (int64_t p = 0; p < nq; ++p) {
      if (!R || !taken) continue;
      const int64_t q = qsel ? qsel[p] : p;
      if (q < 0 || q >= N) {
#pragma omp atomic write
        bad = 1;
        continue;
      }
      for (int64_t i = 0; i < m; ++i) {
        R[i] = dot(Q + q * d, Ql + i * d, d);
        taken[i] = 0;
      }
      /* s rounds of the single-expert rule over the landmarks left */
      for (int64_t j = 0; j < s; ++j) {
        int64_t best = -1;
        for (int64_t i = 0; i < m; ++i) {
          if (taken[i]) continue;
          if (best < 0 || R[i] > R[best]) best = i; /* strict: first maximum */
        }
        taken[best] = 1;
        routes[p * s + j] = (int32_t)best;
      }
    }
    free(R);
    free(taken);
  }
  return bad == 2 ? -2 : (bad ? -1 : 0);
}

int mita_oracle_bucket_s(const int32_t* routes, int64_t N, int64_t m, int64_t s,
                         int32_t* offsets, int32_t* perm) {
  if (!routes || !offsets || !perm || N < 1 || m < 1 || s < 1 || s > m) return -1;
  for (int64_t e = 0; e <= m; ++e) offsets[e] = 0;
  for (int64_t q = 0; q < N; ++q)
    for (int64_t j = 0; j < s; ++j) {
      const int32_t e = routes[q * s + j];
      if (e < 0 || e >= m) return -1;
      for (int64_t i = 0; i < j; ++i)
        if (routes[q * s + i] == e) return -1; /* experts of a query are distinct */
      offsets[e + 1] += 1;
    }
  for (int64_t e = 0; e < m; ++e) offsets[e + 1] += offsets[e];
  int32_t* fill = (int32_t*)malloc((size_t)m * sizeof(int32_t));
  if (!fill) return -2;
  for (int64_t e = 0; e < m; ++e) fill[e] = offsets[e];
  /* queries in increasing index: each expert's group stays in index order */
  for (int64_t q = 0; q < N; ++q)
    for (int64_t j = 0; j < s; ++j) perm[fill[routes[q * s + j]]++] = (int32_t)q;
  free(fill);
  return 0;
}

int mita_oracle_output_s(const double* Q, const double* K, const double* V, const double* Ql,
                         const double* Vl, const int32_t* idx, const int32_t* routes, int64_t N,
                         int64_t d, int64_t m, int64_t k, int64_t s, double scale,
                         const int64_t* qsel, int64_t nq, double* out) {
  if (!Q || !K || !V || !Ql || !Vl || !idx || !routes || !out) return -1;
  if (N < 1 || d < 1 || m < 1 || k < 1 || k > N || s < 1 || s > m) return -1;
  if (!(scale > 0.0) || isinf(scale)) return -1;
  if (!qsel && nq != N) return -1;
  if (nq < 0) return -1;
  int bad = 0;
#pragma omp parallel
  {
    const int64_t np = m + s * k; /* pairs one query attends over */
    double* w = (double*)malloc((size_t)np * sizeof(double));
    int32_t* key = (int32_t*)malloc((size_t)(s * k) * sizeof(int32_t));
    if (!w || !key) {
#pragma omp atomic write
      bad = 2;
    }
#pragma omp for schedule(static)
    for (int64_t p = 0; p < nq; ++p) {
      if (!w || !key) continue;
      const int64_t q = qsel ? qsel[p] : p;
      int ok = q >= 0 && q < N;
      for (int64_t j = 0; ok && j < s; ++j)
        ok = routes[q * s + j] >= 0 && routes[q * s + j] < m;
      if (!ok) {
#pragma omp atomic write
        bad = 1;
        continue;
      }
      /* the raw keys: expert routes[q][0]'s k keys, then the next expert's */
      for (int64_t j = 0; j < s; ++j)
        for (int64_t t = 0; t < k; ++t)
          key[j * k + t] = idx[(int64_t)routes[q * s + j] * k + t];
      double mx = -INFINITY;
      for (int64_t i = 0; i < m; ++i) {
        w[i] = scale * dot(Q + q * d, Ql + i * d, d);
        if (w[i] > mx) mx = w[i];
      }
      for (int64_t t = 0; t < s * k; ++t) {
        w[m + t] = scale * dot(Q + q * d, K + (int64_t)key[t] * d, d);
        if (w[m + t] > mx) mx = w[m + t];
      }
      double z = 0.0;
      for (int64_t i = 0; i < np; ++i) {
        w[i] = exp(w[i] - mx);
        z += w[i];
      }
      for (int64_t c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int64_t i = 0; i < m; ++i) acc += w[i] * Vl[i * d + c];
        for (int64_t t = 0; t < s * k; ++t) acc += w[m + t] * V[(int64_t)key[t] * d + c];
        out[p * d + c] = acc / z;
      }
    }
    free(w);
    free(key);
  }
  return bad == 2 ? -2 : (bad ? -1 : 0);
}

/* ------------------------------------------------------------------------ */
/* Dense attention (the baseline)                                           */
/* ------------------------------------------------------------------------ */

int mita_oracle_dense(const double* Q, const double* K, const double* V, int64_t N, int64_t d,
                      double scale, const int64_t* qsel, int64_t nq, double* out) {
  if (!Q || !K || !V || !out) return -1;
  if (N < 1 || d < 1) return -1;
  if (!(scale > 0.0) || isinf(scale)) return -1;
  if (!qsel && nq != N) return -1;
  if (nq < 0) return -1;
  int bad = 0;
#pragma omp parallel
  {
    double* w = (double*)malloc((size_t)N * sizeof(double));
    if (!w) {
#pragma omp atomic write
      bad = 2;
    }
#pragma omp for schedule(static)
    for (int64_t p = 0; p < nq; ++p) {
      if (!w) continue;
      const int64_t q = qsel ? qsel[p] : p;
      if (q < 0 || q >= N) {
#pragma omp atomic write
        bad = 1;
        continue;
      }
      /* logits over every key, then one softmax */
      double top = -INFINITY;
      for (int64_t t = 0; t < N; ++t) {
        w[t] = scale * dot(Q + q * d, K + t * d, d);
        if (w[t] > top) top = w[t];
      }
      double total = 0.0;
      for (int64_t t = 0; t < N; ++t) {
        w[t] = exp(w[t] - top);
        total += w[t];
      }
      for (int64_t c = 0; c < d; ++c) {
        double sum = 0.0;
        for (int64_t t = 0; t < N; ++t) sum += w[t] * V[t * d + c];
        out[p * d + c] = sum / total;
      }
    }
    free(w);
  }
  return bad == 2 ? -2 : (bad ? -1 : 0);
}

/* ------------------------------------------------------------------------ */
/* All steps over B*H slices                                                 */
/* ------------------------------------------------------------------------ */

int mita_oracle_forward(const double* Q, const double* K, const double* V, int64_t B,
                        int64_t H, int64_t N, int64_t d, int64_t gh, int64_t gw, int64_t mh,
                        int64_t mw, int64_t k, double scale, int round_mode, double* out,
                        int32_t* idx, int32_t* route, double* Ql, double* Vl,
                        int32_t* offsets, int32_t* perm) {
  if (!Q || !K || !V || !out || !idx || !route || B < 1 || H < 1) return -1;
  const int64_t m = mh * mw;
  double* ql = (double*)malloc((size_t)(m * d) * sizeof(double));
  double* vl = (double*)malloc((size_t)(m * d) * sizeof(double));
  int32_t* off = (int32_t*)malloc((size_t)(m + 1) * sizeof(int32_t));
  int32_t* pm = (int32_t*)malloc((size_t)N * sizeof(int32_t));
  int rc = (ql && vl && off && pm) ? 0 : -2;
  for (int64_t s = 0; s < B * H && rc == 0; ++s) {
    const double* q = Q + s * N * d;
    const double* kk = K + s * N * d;
    const double* v = V + s * N * d;
    int32_t* ix = idx + s * m * k;
    int32_t* rt = route + s * N;
    rc = mita_oracle_pool(q, N, d, gh, gw, mh, mw, round_mode, ql);
    if (rc == 0) rc = mita_oracle_topk(ql, kk, N, d, m, k, ix, NULL);
    if (rc == 0) rc = mita_oracle_landmark_values(ql, kk, v, N, d, m, scale, vl);
    if (rc == 0) rc = mita_oracle_route(q, ql, N, d, m, NULL, N, rt, NULL);
    if (rc == 0) rc = mita_oracle_bucket(rt, N, m, off, pm);
    if (rc == 0)
      rc = mita_oracle_output(q, kk, v, ql, vl, ix, rt, N, d, m, k, scale, NULL, N,
                              out + s * N * d);
    if (rc == 0) {
      if (Ql) memcpy(Ql + s * m * d, ql, (size_t)(m * d) * sizeof(double));
      if (Vl) memcpy(Vl + s * m * d, vl, (size_t)(m * d) * sizeof(double));
      if (offsets) memcpy(offsets + s * (m + 1), off, (size_t)(m + 1) * sizeof(int32_t));
      if (perm) memcpy(perm + s * N, pm, (size_t)N * sizeof(int32_t));
    }
  }
  free(ql);
  free(vl);
  free(off);
  free(pm);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Backward pass (training): gradients of sum(dout * out) with respect to    */
/* Q, K and V, the experts and routes held fixed                              */
/* ------------------------------------------------------------------------ */

int mita_oracle_backward(const double* Q, const double* K, const double* V, int64_t N,
                         int64_t d, int64_t gh, int64_t gw, int64_t mh, int64_t mw, int64_t k,
                         double scale, int round_mode, const int32_t* idx, const int32_t* route,
                         const double* dout, double* dQ, double* dK, double* dV) {
  const int64_t m = mh * mw;
  if (!Q || !K || !V || !idx || !route || !dout || !dQ || !dK || !dV) return -1;
  if (N < 1 || d < 1 || m < 1 || m > N || k < 1 || k > N) return -1;
  if (!(scale > 0.0) || isinf(scale)) return -1;
  double* Ql = (double*)calloc((size_t)(m * d), sizeof(double));
  double* Vl = (double*)calloc((size_t)(m * d), sizeof(double));
  double* dQl = (double*)calloc((size_t)(m * d), sizeof(double));
  double* dVl = (double*)calloc((size_t)(m * d), sizeof(double));
  double* w = (double*)malloc((size_t)((m + k > N ? m + k : N) * 2) * sizeof(double));
  int rc = (Ql && Vl && dQl && dVl && w) ? 0 : -2;
  /* the forward's landmark queries and values (the same functions as the
   * forward pass; the rounding of Ql is taken as the identity below) */
  if (rc == 0) rc = mita_oracle_pool(Q, N, d, gh, gw, mh, mw, round_mode, Ql);
  if (rc == 0) rc = mita_oracle_landmark_values(Ql, K, V, N, d, m, scale, Vl);
  if (rc == 0) {
    for (int64_t i = 0; i < N * d; ++i) dQ[i] = dK[i] = dV[i] = 0.0;
    double* dw = w + (m + k > N ? m + k : N);
    /* 1. the output softmax of each query over its m + k pairs */
    for (int64_t q = 0; q < N && rc == 0; ++q) {
      const int64_t e = route[q];
      if (e < 0 || e >= m) {
        rc = -1;
        break;
      }
      const int32_t* ex = idx + e * k;
      const double* qq = Q + q * d;
      const double* G = dout + q * d;
      double mx = -INFINITY;
      for (int64_t i = 0; i < m; ++i) {
        w[i] = scale * dot(qq, Ql + i * d, d);
        if (w[i] > mx) mx = w[i];
      }
      for (int64_t j = 0; j < k; ++j) {
        w[m + j] = scale * dot(qq, K + (int64_t)ex[j] * d, d);
        if (w[m + j] > mx) mx = w[m + j];
      }
      double z = 0.0;
      for (int64_t i = 0; i < m + k; ++i) {
        w[i] = exp(w[i] - mx);
        z += w[i];
      }
      for (int64_t i = 0; i < m + k; ++i) w[i] /= z; /* the softmax weights */
      /* dw: the gradient of each weight (dout . its value) */
      double c = 0.0;
      for (int64_t i = 0; i < m; ++i) {
        dw[i] = dot(G, Vl + i * d, d);
        c += w[i] * dw[i];
      }
      for (int64_t j = 0; j < k; ++j) {
        dw[m + j] = dot(G, V + (int64_t)ex[j] * d, d);
        c += w[m + j] * dw[m + j];
      }
      /* through the softmax to the logits, then to the dot products */
      for (int64_t i = 0; i < m; ++i) {
        const double g = scale * w[i] * (dw[i] - c);
        for (int64_t a = 0; a < d; ++a) {
          dQ[q * d + a] += g * Ql[i * d + a];
          dQl[i * d + a] += g * qq[a];
          dVl[i * d + a] += w[i] * G[a];
        }
      }
      for (int64_t j = 0; j < k; ++j) {
        const int64_t t = ex[j];
        const double g = scale * w[m + j] * (dw[m + j] - c);
        for (int64_t a = 0; a < d; ++a) {
          dQ[q * d + a] += g * K[t * d + a];
          dK[t * d + a] += g * qq[a];
          dV[t * d + a] += w[m + j] * G[a];
        }
      }
    }
    /* 2. the landmarks' cross-attention over all N keys (Vl = softmax(scale
     *    Ql K^T) V) */
    for (int64_t i = 0; i < m && rc == 0; ++i) {
      double mx = -INFINITY;
      for (int64_t t = 0; t < N; ++t) {
        w[t] = scale * dot(Ql + i * d, K + t * d, d);
        if (w[t] > mx) mx = w[t];
      }
      double z = 0.0;
      for (int64_t t = 0; t < N; ++t) {
        w[t] = exp(w[t] - mx);
        z += w[t];
      }
      double c = 0.0;
      for (int64_t t = 0; t < N; ++t) {
        w[t] /= z;
        dw[t] = dot(dVl + i * d, V + t * d, d);
        c += w[t] * dw[t];
      }
      for (int64_t t = 0; t < N; ++t) {
        const double g = scale * w[t] * (dw[t] - c);
        for (int64_t a = 0; a < d; ++a) {
          dQl[i * d + a] += g * K[t * d + a];
          dK[t * d + a] += g * Ql[i * d + a];
          dV[t * d + a] += w[t] * dVl[i * d + a];
        }
      }
    }
    /* 3. the pooling: Ql[i] is the mean of Q over window i */
    for (int64_t i = 0; i < m && rc == 0; ++i) {
      int64_t r0, r1, c0, c1;
      rc = mita_oracle_window(gh, gw, mh, mw, i, &r0, &r1, &c0, &c1);
      if (rc != 0) break;
      const double cnt = (double)((r1 - r0) * (c1 - c0));
      for (int64_t r = r0; r < r1; ++r)
        for (int64_t cc = c0; cc < c1; ++cc) {
          const int64_t t = r * gw + cc;
          for (int64_t a = 0; a < d; ++a) dQ[t * d + a] += dQl[i * d + a] / cnt;
        }
    }
  }
  free(Ql);
  free(Vl);
  free(dQl);
  free(dVl);
  free(w);
  return rc;
}
