/*
 * oracle.c -- plain, slow fp64 CPU reference for the EntmaxKV decode path.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path.  It shares no code,
 * header, table or constant generator with the HIP library.
 *
 * "The EntmaxKV summary" = "Resumen Tecnico: EntmaxKV - Decodificacion
 * Consciente del Soporte para Atencion Entmax" (gist.science/es/paper/
 * 2605.21649).  Section numbers below are that page's.  Where the page is
 * silent the reading taken is stated at the function.
 *
 * Every floating-point step is written in the order the definition states;
 * the only parallelism is an OpenMP loop over independent (batch, head) rows,
 * which does not change any arithmetic.  Build with -ffp-contract=off.
 */
#include "oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* element access and storage rounding                                       */
/* ------------------------------------------------------------------------ */

static double ld(const void *p, int dtype, size_t i) {
  if (dtype == 0) return (double)((const float *)p)[i];
  uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round-to-nearest-even of x to bfloat16 (8 significant bits, float32 exponent
 * range, subnormal quantum 2^-133), done directly from the fp64 value. */
double orc_round_bf16(double x) {
  if (isnan(x) || isinf(x) || x == 0.0) return x;
  int e;
  frexp(x, &e); /* |x| = m 2^e, 0.5 <= m < 1 */
  int qexp = (e < -125 ? -125 : e) - 8;
  double r = nearbyint(ldexp(x, -qexp)); /* default rounding mode: ties to even */
  double y = ldexp(r, qexp);
  const double maxbf = ldexp(255.0, 120);
  if (fabs(y) > maxbf) return x > 0 ? INFINITY : -INFINITY;
  return y;
}

/* OCP 8-bit floating point, E4M3 ("FN": no infinities).  Code = s eeee mmm,
 * exponent bias 7: e = 0 gives the subnormals m/8 * 2^-6, otherwise
 * (1 + m/8) * 2^(e-7); e = 15, m = 7 is NaN, so the largest finite value is
 * 448.  This is the format of the compact metadata's mean and variance. */
double orc_e4m3_decode(uint8_t c) {
  int sgn = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m / 8.0, -6);
  else v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sgn ? -v : v;
}

/* Nearest E4M3 code to x, ties to the even code (mantissa bit 0 clear),
 * magnitudes beyond the largest finite value saturate to +-448, NaN gives the
 * NaN code.  Done by binary search over the 127 non-negative finite codes,
 * whose values increase with the code. */
uint8_t orc_e4m3_encode(double x) {
  if (isnan(x)) return 0x7F;
  uint8_t sgn = signbit(x) ? 0x80 : 0x00;
  double a = fabs(x);
  if (a >= 448.0) return (uint8_t)(sgn | 0x7E);
  int lo = 0, hi = 0x7E; /* decode(lo) <= a < decode(hi) */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (orc_e4m3_decode((uint8_t)mid) <= a) lo = mid; else hi = mid;
  }
  double dl = a - orc_e4m3_decode((uint8_t)lo), dh = orc_e4m3_decode((uint8_t)hi) - a;
  int c = (dl < dh) ? lo : (dh < dl) ? hi : ((lo & 1) == 0 ? lo : hi);
  return (uint8_t)(sgn | c);
}

static void store_val(void *p, int dtype, size_t i, double x) {
  if (dtype == 0) {
    ((float *)p)[i] = (float)x; /* RNE */
  } else {
    float f = (float)orc_round_bf16(x); /* exact: already a bf16 value */
    uint32_t u;
    memcpy(&u, &f, 4);
    ((uint16_t *)p)[i] = (uint16_t)(u >> 16);
  }
}

double orc_round_f32(double x) { return (double)(float)x; }

double orc_round_f32_up(double x) {
  if (isnan(x)) return x;
  float f = (float)x;
  if ((double)f < x) f = nextafterf(f, INFINITY);
  return (double)f;
}

static double cscale(const orc_shape *s) { return s->scale != 0.0 ? s->scale : 1.0 / sqrt((double)s->d); }

static int32_t n_pages(const orc_shape *s, int32_t L) {
  if (L <= 0) return 0;
  int32_t n = (L + s->P - 1) / s->P;
  return n > s->max_pages ? s->max_pages : n;
}

static int32_t seq_len(const orc_shape *s, const int32_t *seq_lens, int b) {
  int32_t L = seq_lens[b];
  if (L < 0) L = 0;
  int64_t cap = (int64_t)s->max_pages * s->P;
  return (int64_t)L > cap ? (int32_t)cap : L;
}

static int32_t page_fill(const orc_shape *s, int32_t L, int32_t p) {
  int32_t n = L - p * s->P;
  return n > s->P ? s->P : n;
}

/* ------------------------------------------------------------------------ */
/* Gauss-Hermite nodes: Golub-Welsch (eigenvalues of the Jacobi matrix of the  */
/* Hermite recurrence, by cyclic Jacobi rotations), then each node polished by */
/* Newton on H_16 and weighted by the classical closed form                    */
/*   w = 2^(n-1) n! sqrt(pi) / (n^2 H_{n-1}(x)^2).                             */
/* ------------------------------------------------------------------------ */

static void hermite_h(int n, double x, double *hn, double *hn1) {
  /* physicists' recurrence H_{k+1} = 2x H_k - 2k H_{k-1} */
  double h0 = 1.0, h1 = 2.0 * x;
  if (n == 0) { *hn = h0; *hn1 = 0.0; return; }
  for (int k = 1; k < n; ++k) {
    double h2 = 2.0 * x * h1 - 2.0 * k * h0;
    h0 = h1;
    h1 = h2;
  }
  *hn = h1;
  *hn1 = h0;
}

void orc_gauss_hermite16(double *nodes, double *weights) {
  enum { N = 16 };
  double A[N][N], V[N][N];
  memset(A, 0, sizeof A);
  for (int i = 0; i < N; ++i)
    for (int j = 0; j < N; ++j) V[i][j] = (i == j);
  for (int k = 1; k < N; ++k) A[k - 1][k] = A[k][k - 1] = sqrt(k / 2.0);
  for (int sweep = 0; sweep < 100; ++sweep) {
    double off = 0.0;
    for (int p = 0; p < N; ++p)
      for (int q = p + 1; q < N; ++q) off += A[p][q] * A[p][q];
    if (off < 1e-60) break;
    for (int p = 0; p < N; ++p)
      for (int q = p + 1; q < N; ++q) {
        if (A[p][q] == 0.0) continue;
        double theta = (A[q][q] - A[p][p]) / (2.0 * A[p][q]);
        double t = (theta >= 0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
        double c = 1.0 / sqrt(t * t + 1.0), sn = t * c;
        for (int k = 0; k < N; ++k) { /* A <- A J */
          double akp = A[k][p], akq = A[k][q];
          A[k][p] = c * akp - sn * akq;
          A[k][q] = sn * akp + c * akq;
        }
        for (int k = 0; k < N; ++k) { /* A <- J^T A */
          double apk = A[p][k], aqk = A[q][k];
          A[p][k] = c * apk - sn * aqk;
          A[q][k] = sn * apk + c * aqk;
        }
        for (int k = 0; k < N; ++k) {
          double vkp = V[k][p], vkq = V[k][q];
          V[k][p] = c * vkp - sn * vkq;
          V[k][q] = sn * vkp + c * vkq;
        }
      }
  }
  double x[N];
  for (int i = 0; i < N; ++i) x[i] = A[i][i];
  for (int i = 1; i < N; ++i) /* insertion sort ascending */
    for (int j = i; j > 0 && x[j - 1] > x[j]; --j) { double t = x[j]; x[j] = x[j - 1]; x[j - 1] = t; }
  double fact = 1.0;
  for (int k = 2; k <= N; ++k) fact *= k;
  const double num = ldexp(1.0, N - 1) * fact * sqrt(M_PI) / ((double)N * N);
  for (int i = 0; i < N; ++i) {
    double xi = x[i];
    for (int it = 0; it < 5; ++it) { /* Newton: H_n' = 2n H_{n-1} */
      double hn, hn1;
      hermite_h(N, xi, &hn, &hn1);
      double step = hn / (2.0 * N * hn1);
      xi -= step;
      if (fabs(step) < 1e-17 * (1.0 + fabs(xi))) break;
    }
    double hn, hn1;
    hermite_h(N, xi, &hn, &hn1);
    nodes[i] = xi;
    weights[i] = num / (hn1 * hn1);
  }
}

/* ------------------------------------------------------------------------ */
/* build_page_meta -- EntmaxKV summary 2.A: per-page, per-coordinate key        */
/* bounding box (k_min, k_max) and Gaussian statistics (first and second        */
/* moments: mean and variance).  Reading: population variance (divisor n) over  */
/* the filled slots, var = max(0, S2/n - mean^2) from fp64 sums, each stored    */
/* value rounded once to the metadata dtype.                                    */
/* ------------------------------------------------------------------------ */
/* Compact records (fmt 1, bf16 keys only): k_min and k_max as above, mean and */
/* var each rounded once to E4M3 (nearest, ties to even, saturating), record   */
/* = k_min bf16[d] | k_max bf16[d] | mean e4m3[d] | var e4m3[d] (6d bytes).    */
static void build_meta(const orc_shape *s, const void *k_pool, const int32_t *page_table,
                       const int32_t *seq_lens, const int32_t *from_token, void *meta, int fmt) {
  const int d = s->d, P = s->P, Hkv = s->Hkv;
  for (int b = 0; b < s->B; ++b) {
    int32_t L = seq_len(s, seq_lens, b);
    int32_t np = n_pages(s, L);
    int32_t first = 0;
    if (from_token) {
      int32_t f = from_token[b] < 0 ? 0 : from_token[b];
      first = f / P;
    }
#pragma omp parallel for schedule(dynamic, 16)
    for (int32_t p = first; p < np; ++p) {
      int32_t phys = page_table[(size_t)b * s->max_pages + p];
      if (phys < 0 || phys >= s->num_phys) continue;
      int32_t n = page_fill(s, L, p);
      for (int g = 0; g < Hkv; ++g) {
        size_t kbase = (((size_t)phys * Hkv + g) * P) * d;
        size_t mbase = (((size_t)phys * Hkv + g) * 4) * d;
        for (int i = 0; i < d; ++i) {
          double kmin = INFINITY, kmax = -INFINITY, s1 = 0.0, s2 = 0.0;
          for (int j = 0; j < n; ++j) {
            double k = ld(k_pool, s->dtype, kbase + (size_t)j * d + i);
            if (k < kmin) kmin = k;
            if (k > kmax) kmax = k;
            s1 += k;
            s2 += k * k;
          }
          double mean = s1 / n;
          double var = s2 / n - mean * mean;
          if (!(var > 0.0)) var = 0.0;
          if (fmt == 0) {
            store_val(meta, s->dtype, mbase + 0 * d + i, kmin);
            store_val(meta, s->dtype, mbase + 1 * d + i, kmax);
            store_val(meta, s->dtype, mbase + 2 * d + i, mean);
            store_val(meta, s->dtype, mbase + 3 * d + i, var);
          } else {
            uint8_t *rec = (uint8_t *)meta + ((size_t)phys * Hkv + g) * (size_t)(6 * d);
            store_val(rec, 1, (size_t)i, kmin);
            store_val(rec, 1, (size_t)d + i, kmax);
            rec[4 * d + i] = orc_e4m3_encode(mean);
            rec[5 * d + i] = orc_e4m3_encode(var);
          }
        }
      }
    }
  }
}

void orc_build_page_meta(const orc_shape *s, const void *k_pool, const int32_t *page_table,
                         const int32_t *seq_lens, const int32_t *from_token, void *meta) {
  build_meta(s, k_pool, page_table, seq_lens, from_token, meta, 0);
}

void orc_build_page_meta_f8(const orc_shape *s, const void *k_pool, const int32_t *page_table,
                            const int32_t *seq_lens, const int32_t *from_token, void *meta) {
  build_meta(s, k_pool, page_table, seq_lens, from_token, meta, 1);
}

/* ------------------------------------------------------------------------ */
/* score_pages -- EntmaxKV summary 2.A.                                         */
/*  box  = c sum_i max(q_i kmin_i, q_i kmax_i)  (deterministic upper bound on   */
/*         every score in the page), stored rounded toward +infinity;           */
/*  mu   = c sum_i q_i mean_i,   var = c^2 sum_i q_i^2 var_i  (Gaussian model    */
/*         of the page's scores, diagonal reading), stored round-to-nearest.    */
/* ------------------------------------------------------------------------ */
static int row_count(const orc_shape *s, const int32_t *rows, int32_t n_rows) {
  return rows ? n_rows : s->B * s->Hq;
}
static int row_at(const int32_t *rows, int i) { return rows ? rows[i] : i; }

/* Compact records: the stored mean and variance are E4M3 values, decoded      */
/* exactly; the products with q (bf16) remain exact in fp64.                    */
static double meta_at(const orc_shape *s, const void *meta, int32_t phys, int g, int kind, int i,
                      int fmt) {
  const int d = s->d;
  if (fmt == 0) return ld(meta, s->dtype, (((size_t)phys * s->Hkv + g) * 4 + kind) * d + i);
  const uint8_t *rec = (const uint8_t *)meta + ((size_t)phys * s->Hkv + g) * (size_t)(6 * d);
  if (kind < 2) return ld(rec, 1, (size_t)kind * d + i);
  return orc_e4m3_decode(rec[(size_t)(4 + (kind - 2)) * d + i]);
}

static void score_pages(const orc_shape *s, const void *q, const void *meta,
                        const int32_t *page_table, const int32_t *seq_lens,
                        const int32_t *rows, int32_t n_rows, float *box, float *mu, float *var,
                        int fmt) {
  const int d = s->d, G = s->Hq / s->Hkv;
  const double c = cscale(s);
  const double c2 = c * c;
  int nr = row_count(s, rows, n_rows);
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < nr; ++r) {
    int row = row_at(rows, r), b = row / s->Hq, h = row % s->Hq, g = h / G;
    int32_t L = seq_len(s, seq_lens, b);
    int32_t np = n_pages(s, L);
    for (int32_t p = 0; p < np; ++p) {
      size_t o = (size_t)row * s->max_pages + p;
      int32_t phys = page_table[(size_t)b * s->max_pages + p];
      if (phys < 0 || phys >= s->num_phys) {
        box[o] = NAN; mu[o] = NAN; var[o] = NAN;
        continue;
      }
      double sb = 0.0, sm = 0.0, sv = 0.0;
      for (int i = 0; i < d; ++i) {
        double qi = ld(q, s->dtype, (size_t)row * d + i);
        double a = qi * meta_at(s, meta, phys, g, 0, i, fmt);
        double bb = qi * meta_at(s, meta, phys, g, 1, i, fmt);
        sb += (a > bb ? a : bb);
        sm += qi * meta_at(s, meta, phys, g, 2, i, fmt);
        sv += (qi * qi) * meta_at(s, meta, phys, g, 3, i, fmt);
      }
      box[o] = (float)orc_round_f32_up(c * sb);
      mu[o] = (float)(c * sm);
      var[o] = (float)(c2 * sv);
    }
  }
}

void orc_score_pages(const orc_shape *s, const void *q, const void *meta,
                     const int32_t *page_table, const int32_t *seq_lens,
                     const int32_t *rows, int32_t n_rows, float *box, float *mu, float *var) {
  score_pages(s, q, meta, page_table, seq_lens, rows, n_rows, box, mu, var, 0);
}

void orc_score_pages_f8(const orc_shape *s, const void *q, const void *meta,
                        const int32_t *page_table, const int32_t *seq_lens,
                        const int32_t *rows, int32_t n_rows, float *box, float *mu, float *var) {
  score_pages(s, q, meta, page_table, seq_lens, rows, n_rows, box, mu, var, 1);
}

/* ------------------------------------------------------------------------ */
/* select_pages_topk -- EntmaxKV summary 2.B.1: the k pages with the highest    */
/* bounding-box bounds.  Readings: ties go to the lower logical page index, a   */
/* NaN bound ranks below every number, N_b <= k keeps every page, and the       */
/* result is listed in ascending page order.                                    */
/* ------------------------------------------------------------------------ */
typedef struct { double key; int32_t idx; } kv_pair;

static int cmp_desc(const void *a, const void *b) {
  const kv_pair *x = (const kv_pair *)a, *y = (const kv_pair *)b;
  if (x->key > y->key) return -1;
  if (x->key < y->key) return 1;
  return (x->idx > y->idx) - (x->idx < y->idx);
}
static int cmp_int(const void *a, const void *b) {
  int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
  return (x > y) - (x < y);
}

void orc_select_topk(const orc_shape *s, const float *box, const int32_t *seq_lens, int32_t k,
                     const uint8_t *seq_mask, const int32_t *rows, int32_t n_rows,
                     int32_t *sel_idx, int32_t *sel_cnt) {
  int nr = row_count(s, rows, n_rows);
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < nr; ++r) {
    int row = row_at(rows, r), b = row / s->Hq;
    if (seq_mask && !seq_mask[b]) continue;
    int32_t np = n_pages(s, seq_len(s, seq_lens, b));
    kv_pair *v = (kv_pair *)malloc(sizeof(kv_pair) * (np > 0 ? np : 1));
    for (int32_t p = 0; p < np; ++p) {
      double x = box[(size_t)row * s->max_pages + p];
      v[p].key = isnan(x) ? -INFINITY : x;
      v[p].idx = p;
    }
    qsort(v, np, sizeof(kv_pair), cmp_desc);
    int32_t m = np < k ? np : k;
    int32_t *out = sel_idx + (size_t)row * s->max_pages;
    for (int32_t i = 0; i < m; ++i) out[i] = v[i].idx;
    qsort(out, m, sizeof(int32_t), cmp_int);
    sel_cnt[row] = m;
    free(v);
  }
}

/* ------------------------------------------------------------------------ */
/* select_pages_gauss -- EntmaxKV summary 2.B.2: estimate the global entmax     */
/* threshold from the page Gaussians by solving an approximate normalization    */
/* equation, then keep the pages whose estimated maximum score reaches the      */
/* threshold lowered by a safety margin Delta.                                  */
/* Readings (the page gives no formulas):                                       */
/*  * normalization equation: F(tau) = 1 with                                   */
/*      F(tau) = sum_p n_p sum_j w_j [(alpha-1)(mu_p + sqrt2 sigma_p x_j) - tau]_+^(1/(alpha-1))  */
/*    the 16-point Gauss-Hermite form (w_j = GH weight / sqrt(pi)) of            */
/*    sum_p n_p E[((alpha-1)s - tau)_+^(1/(alpha-1))], s ~ N(mu_p, sigma_p^2);   */
/*  * tau_hat = the bisection limit "lo" with F(lo) >= 1;                        */
/*  * estimated maximum score = min(mu_p + n_sigma sigma_p, box_p);             */
/*  * keep p iff est_p >= tau_hat/(alpha-1) - Delta (score units);               */
/*  * pages with a non-finite box/mu/var are ignored; if nothing is kept the    */
/*    page of largest est_p (lowest index on ties) is kept.                     */
/* ------------------------------------------------------------------------ */
typedef struct { double mu, sig, s2, box; int32_t n; int ok; } gpage;

static double gauss_F(const gpage *pg, int32_t np, double a, double beta, const double *x,
                      const double *w, double tau) {
  const double sqrt2 = sqrt(2.0);
  double F = 0.0;
  for (int32_t p = 0; p < np; ++p) {
    if (!pg[p].ok) continue;
    double inner = 0.0;
    for (int j = 0; j < 16; ++j) {
      double v = a * (pg[p].mu + sqrt2 * pg[p].sig * x[j]) - tau;
      if (v > 0.0) inner += w[j] * pow(v, beta);
    }
    F += pg[p].n * inner;
  }
  return F;
}

/* F(tau) over an explicit page list (exposed for pins). */
double orc_gauss_mass(const float *mu, const float *var, const int32_t *n, int32_t np, double alpha,
                      double tau) {
  double x[16], w[16];
  orc_gauss_hermite16(x, w);
  for (int j = 0; j < 16; ++j) w[j] /= sqrt(M_PI);
  gpage *pg = (gpage *)malloc(sizeof(gpage) * (np > 0 ? np : 1));
  for (int32_t p = 0; p < np; ++p) {
    pg[p].ok = isfinite(mu[p]) && isfinite(var[p]);
    pg[p].mu = mu[p];
    pg[p].s2 = var[p] > 0.0f ? var[p] : 0.0;
    pg[p].sig = sqrt(pg[p].s2);
    pg[p].box = INFINITY;
    pg[p].n = n[p];
  }
  double F = gauss_F(pg, np, alpha - 1.0, 1.0 / (alpha - 1.0), x, w, tau);
  free(pg);
  return F;
}

void orc_select_gauss(const orc_shape *s, const float *box, const float *mu, const float *var,
                      const int32_t *seq_lens, double alpha, double delta, double n_sigma,
                      const uint8_t *seq_mask, const int32_t *rows, int32_t n_rows,
                      int32_t *sel_idx, int32_t *sel_cnt, double *tau_hat) {
  double x[16], w[16];
  orc_gauss_hermite16(x, w);
  for (int j = 0; j < 16; ++j) w[j] /= sqrt(M_PI);
  const double a = alpha - 1.0, beta = 1.0 / a;
  const double sqrt2 = sqrt(2.0);
  int nr = row_count(s, rows, n_rows);
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < nr; ++r) {
    int row = row_at(rows, r), b = row / s->Hq;
    if (seq_mask && !seq_mask[b]) continue;
    int32_t L = seq_len(s, seq_lens, b);
    int32_t np = n_pages(s, L);
    int32_t *out = sel_idx + (size_t)row * s->max_pages;
    gpage *pg = (gpage *)malloc(sizeof(gpage) * (np > 0 ? np : 1));
    int any = 0;
    double mu_max = -INFINITY, hi = -INFINITY;
    for (int32_t p = 0; p < np; ++p) {
      size_t o = (size_t)row * s->max_pages + p;
      double m = mu[o], v2 = var[o], bx = box[o];
      pg[p].ok = isfinite(m) && isfinite(v2) && isfinite(bx);
      pg[p].mu = m;
      pg[p].s2 = v2 > 0.0 ? v2 : 0.0;
      pg[p].sig = sqrt(pg[p].s2);
      pg[p].box = bx;
      pg[p].n = page_fill(s, L, p);
      if (!pg[p].ok) continue;
      any = 1;
      if (m > mu_max) mu_max = m;
      double top = a * (m + sqrt2 * pg[p].sig * x[15]);
      if (top > hi) hi = top;
    }
    if (!any) {
      sel_cnt[row] = 0;
      if (tau_hat) tau_hat[row] = NAN;
      free(pg);
      continue;
    }
    /* bracket: F(lo) >= 1, F(hi) = 0 */
    double gap = 1.0, lo = a * mu_max - gap;
    while (gauss_F(pg, np, a, beta, x, w, lo) < 1.0) {
      gap *= 2.0;
      lo = a * mu_max - gap;
    }
    for (;;) {
      double mid = 0.5 * (lo + hi);
      if (mid == lo || mid == hi) break;
      if (gauss_F(pg, np, a, beta, x, w, mid) >= 1.0) lo = mid; else hi = mid;
    }
    if (tau_hat) tau_hat[row] = lo / a;
    double thr = lo / a - delta;
    int32_t cnt = 0;
    for (int32_t p = 0; p < np; ++p) {
      if (!pg[p].ok) continue;
      double dd = thr - pg[p].mu;
      int gauss_ok = (dd <= 0.0) || (n_sigma * n_sigma * pg[p].s2 >= dd * dd);
      if (gauss_ok && pg[p].box >= thr) out[cnt++] = p;
    }
    if (cnt == 0) {
      int32_t best = -1;
      double be = -INFINITY;
      for (int32_t p = 0; p < np; ++p) {
        if (!pg[p].ok) continue;
        double e1 = pg[p].mu + n_sigma * pg[p].sig;
        double est = e1 < pg[p].box ? e1 : pg[p].box;
        if (best < 0 || est > be) { be = est; best = p; }
      }
      out[cnt++] = best;
    }
    sel_cnt[row] = cnt;
    free(pg);
  }
}

/* ------------------------------------------------------------------------ */
/* Group-shared selection: one kept set per KV head, for the G query heads    */
/* that read it.  A variant the EntmaxKV summary leaves open (its policies,    */
/* section 2.B, are stated per query).  Readings:                              */
/*  * Top-k: a page's group score is the largest box over the G heads (a NaN  */
/*    box ranks below every number, as in select_pages_topk); the k pages     */
/*    with the largest group scores, ties to the lower page, ascending list;  */
/*  * Gaussian: a page is kept for the group iff at least one of the G heads  */
/*    keeps it (each head with its own tau_hat, margin and fallback page),    */
/*    i.e. the largest per-head margin est_p - threshold is >= 0.             */
/* rows: optional list of group rows b*Hkv + g (NULL = all).  Outputs are     */
/* [B][Hkv][max_pages] and [B][Hkv]; tau_hat (nullable) [B][Hq] receives the  */
/* heads of the listed groups.                                                 */
/* ------------------------------------------------------------------------ */
void orc_select_topk_group(const orc_shape *s, const float *box, const int32_t *seq_lens, int32_t k,
                           const uint8_t *seq_mask, const int32_t *rows, int32_t n_rows,
                           int32_t *sel_idx, int32_t *sel_cnt) {
  const int G = s->Hq / s->Hkv;
  int nr = rows ? n_rows : s->B * s->Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < nr; ++r) {
    int grow = rows ? rows[r] : r, b = grow / s->Hkv, g = grow % s->Hkv;
    if (seq_mask && !seq_mask[b]) continue;
    int32_t np = n_pages(s, seq_len(s, seq_lens, b));
    kv_pair *v = (kv_pair *)malloc(sizeof(kv_pair) * (np > 0 ? np : 1));
    for (int32_t p = 0; p < np; ++p) {
      double key = -INFINITY;
      for (int h = 0; h < G; ++h) {
        double x = box[((size_t)b * s->Hq + (size_t)g * G + h) * s->max_pages + p];
        if (!isnan(x) && x > key) key = x;
      }
      v[p].key = key;
      v[p].idx = p;
    }
    qsort(v, np, sizeof(kv_pair), cmp_desc);
    int32_t m = np < k ? np : k;
    int32_t *out = sel_idx + (size_t)grow * s->max_pages;
    for (int32_t i = 0; i < m; ++i) out[i] = v[i].idx;
    qsort(out, m, sizeof(int32_t), cmp_int);
    sel_cnt[grow] = m;
    free(v);
  }
}

void orc_select_gauss_group(const orc_shape *s, const float *box, const float *mu, const float *var,
                            const int32_t *seq_lens, double alpha, double delta, double n_sigma,
                            const uint8_t *seq_mask, const int32_t *rows, int32_t n_rows,
                            int32_t *sel_idx, int32_t *sel_cnt, double *tau_hat) {
  const int G = s->Hq / s->Hkv;
  const int MP = s->max_pages;
  int nr = rows ? n_rows : s->B * s->Hkv;
  int32_t *hrows = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nr > 0 ? nr : 1) * G);
  for (int r = 0; r < nr; ++r) {
    int grow = rows ? rows[r] : r, b = grow / s->Hkv, g = grow % s->Hkv;
    for (int h = 0; h < G; ++h) hrows[(size_t)r * G + h] = b * s->Hq + g * G + h;
  }
  int32_t *hs = (int32_t *)malloc(sizeof(int32_t) * (size_t)s->B * s->Hq * MP);
  int32_t *hc = (int32_t *)malloc(sizeof(int32_t) * (size_t)s->B * s->Hq);
  orc_select_gauss(s, box, mu, var, seq_lens, alpha, delta, n_sigma, seq_mask, hrows, nr * G, hs, hc,
                   tau_hat);
  for (int r = 0; r < nr; ++r) {
    int grow = rows ? rows[r] : r, b = grow / s->Hkv;
    if (seq_mask && !seq_mask[b]) continue;
    int32_t np = n_pages(s, seq_len(s, seq_lens, b));
    uint8_t *kept = (uint8_t *)calloc((size_t)(np > 0 ? np : 1), 1);
    for (int h = 0; h < G; ++h) {
      int32_t row = hrows[(size_t)r * G + h];
      for (int32_t i = 0; i < hc[row]; ++i) kept[hs[(size_t)row * MP + i]] = 1;
    }
    int32_t cnt = 0;
    int32_t *out = sel_idx + (size_t)grow * MP;
    for (int32_t p = 0; p < np; ++p)
      if (kept[p]) out[cnt++] = p;
    sel_cnt[grow] = cnt;
    free(kept);
  }
  free(hs);
  free(hc);
  free(hrows);
}

/* ------------------------------------------------------------------------ */
/* alpha-entmax over a reduced set -- EntmaxKV summary 2.C and 3.               */
/* p_t = [(alpha-1)s_t - tau]_+^(1/(alpha-1)) with tau the root of sum p = 1,   */
/* found by bisection on [max X - 1, max X - n^(1-alpha)], X = (alpha-1)s.       */
/* The weights are then divided by their sum (removes the bisection residual). */
/* ------------------------------------------------------------------------ */
static double entmax_F(const double *X, int64_t n, double beta, double tau) {
  double F = 0.0;
  for (int64_t t = 0; t < n; ++t) {
    double v = X[t] - tau;
    if (v > 0.0) F += pow(v, beta);
  }
  return F;
}

static double entmax_tau_X(const double *X, int64_t n, double alpha) {
  const double beta = 1.0 / (alpha - 1.0);
  double mx = -INFINITY;
  for (int64_t t = 0; t < n; ++t) if (X[t] > mx) mx = X[t];
  double lo = mx - 1.0, hi = mx - pow((double)n, 1.0 - alpha);
  for (;;) {
    double mid = 0.5 * (lo + hi);
    if (mid == lo || mid == hi) break;
    if (entmax_F(X, n, beta, mid) >= 1.0) lo = mid; else hi = mid;
  }
  return lo;
}

double orc_entmax_tau(const double *scores, int64_t n, double alpha) {
  double *X = (double *)malloc(sizeof(double) * (n > 0 ? n : 1));
  for (int64_t t = 0; t < n; ++t) X[t] = (alpha - 1.0) * scores[t];
  double tau = entmax_tau_X(X, n, alpha);
  free(X);
  return tau / (alpha - 1.0);
}

static double score_of(const orc_shape *s, const void *q, const void *k_pool, int row, int g,
                       int32_t phys, int j, double c) {
  const int d = s->d;
  size_t kbase = ((((size_t)phys * s->Hkv + g) * s->P) + j) * d;
  double acc = 0.0;
  for (int i = 0; i < d; ++i) acc += ld(q, s->dtype, (size_t)row * d + i) * ld(k_pool, s->dtype, kbase + i);
  return c * acc;
}

void orc_entmax_decode(const orc_shape *s, const void *q, const void *k_pool, const void *v_pool,
                       const int32_t *page_table, const int32_t *seq_lens,
                       const int32_t *sel_idx, const int32_t *sel_cnt, double alpha,
                       const int32_t *rows, int32_t n_rows, double *out, double *tau,
                       double *weights) {
  const int d = s->d, G = s->Hq / s->Hkv, P = s->P;
  const double c = cscale(s), a = alpha - 1.0, beta = 1.0 / a;
  int nr = row_count(s, rows, n_rows);
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < nr; ++r) {
    int row = row_at(rows, r), b = row / s->Hq, h = row % s->Hq, g = h / G;
    int32_t L = seq_len(s, seq_lens, b);
    int32_t np = n_pages(s, L);
    int32_t cnt = sel_idx ? sel_cnt[row] : np;
    double *o = out + (size_t)row * d;
    for (int i = 0; i < d; ++i) o[i] = 0.0;
    if (weights)
      for (size_t t = 0; t < (size_t)s->max_pages * P; ++t) weights[(size_t)row * s->max_pages * P + t] = 0.0;
    /* gather the kept tokens (logical positions ascending) */
    int64_t cap = (int64_t)(cnt > 0 ? cnt : 1) * P;
    double *X = (double *)malloc(sizeof(double) * cap);
    int64_t *pos = (int64_t *)malloc(sizeof(int64_t) * cap);
    int32_t *phs = (int32_t *)malloc(sizeof(int32_t) * cap);
    int64_t n = 0;
    int bad = 0, prev = -1;
    for (int32_t i = 0; i < cnt; ++i) {
      int32_t p = sel_idx ? sel_idx[(size_t)row * s->max_pages + i] : i;
      if (p < 0 || p >= np || p <= prev) { bad = 1; break; }
      prev = p;
      int32_t phys = page_table[(size_t)b * s->max_pages + p];
      if (phys < 0 || phys >= s->num_phys) { bad = 1; break; }
      int32_t fill = page_fill(s, L, p);
      for (int j = 0; j < fill; ++j) {
        X[n] = a * score_of(s, q, k_pool, row, g, phys, j, c);
        pos[n] = (int64_t)p * P + j;
        phs[n] = phys;
        ++n;
      }
    }
    if (bad || n == 0) {
      if (bad) for (int i = 0; i < d; ++i) o[i] = NAN;
      if (tau) tau[row] = NAN;
      free(X); free(pos); free(phs);
      continue;
    }
    double tt = entmax_tau_X(X, n, alpha);
    if (tau) tau[row] = tt / a;
    double Z = 0.0;
    for (int64_t t = 0; t < n; ++t) {
      double v = X[t] - tt;
      X[t] = v > 0.0 ? pow(v, beta) : 0.0;
      Z += X[t];
    }
    for (int64_t t = 0; t < n; ++t) {
      double p = X[t] / Z;
      if (weights) weights[(size_t)row * s->max_pages * P + pos[t]] = p;
      if (p == 0.0) continue;
      int j = (int)(pos[t] % P);
      size_t vbase = ((((size_t)phs[t] * s->Hkv + g) * P) + j) * d;
      for (int i = 0; i < d; ++i) o[i] += p * ld(v_pool, s->dtype, vbase + i);
    }
    free(X); free(pos); free(phs);
  }
}

/* ------------------------------------------------------------------------ */
/* softmax_decode_full -- the full-cache softmax baseline the EntmaxKV summary  */
/* compares against (section 4, efficiency): exact softmax attention over every  */
/* cached token, same score scale.  With a selection (sel_idx, sel_cnt not NULL) */
/* the same softmax runs over the kept pages only: the comparison of section 3   */
/* (under one kept set softmax keeps weight on every discarded token) and of the */
/* approximation-quality results of section 4.  Selection contract as           */
/* orc_entmax_decode, plus: a count outside [0, N_b] makes the row NaN; an empty */
/* kept set gives out = 0 and lse = -inf.                                       */
/* ------------------------------------------------------------------------ */
void orc_softmax_decode(const orc_shape *s, const void *q, const void *k_pool, const void *v_pool,
                        const int32_t *page_table, const int32_t *seq_lens,
                        const int32_t *sel_idx, const int32_t *sel_cnt,
                        const int32_t *rows, int32_t n_rows, double *out, double *lse) {
  const int d = s->d, G = s->Hq / s->Hkv, P = s->P;
  const double c = cscale(s);
  int nr = row_count(s, rows, n_rows);
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < nr; ++r) {
    int row = row_at(rows, r), b = row / s->Hq, h = row % s->Hq, g = h / G;
    int32_t L = seq_len(s, seq_lens, b);
    int32_t np = n_pages(s, L);
    int32_t cnt = sel_idx ? sel_cnt[row] : np;
    double *o = out + (size_t)row * d;
    for (int i = 0; i < d; ++i) o[i] = 0.0;
    int bad = cnt < 0 || cnt > np;
    if (bad) cnt = 0;
    /* the kept tokens: scores, physical pages and slots, page order */
    int64_t cap = (int64_t)(cnt > 0 ? cnt : 1) * P;
    double *S = (double *)malloc(sizeof(double) * cap);
    int32_t *phs = (int32_t *)malloc(sizeof(int32_t) * cap);
    int32_t *slot = (int32_t *)malloc(sizeof(int32_t) * cap);
    int64_t n = 0;
    int32_t prev = -1;
    for (int32_t i = 0; i < cnt && !bad; ++i) {
      int32_t p = sel_idx ? sel_idx[(size_t)row * s->max_pages + i] : i;
      if (p < 0 || p >= np || p <= prev) { bad = 1; break; }
      prev = p;
      int32_t phys = page_table[(size_t)b * s->max_pages + p];
      if (phys < 0 || phys >= s->num_phys) { bad = 1; break; }
      for (int j = 0; j < page_fill(s, L, p); ++j) {
        S[n] = score_of(s, q, k_pool, row, g, phys, j, c);
        phs[n] = phys;
        slot[n] = j;
        ++n;
      }
    }
    if (bad || n == 0) {
      if (bad) for (int i = 0; i < d; ++i) o[i] = NAN;
      if (lse) lse[row] = bad ? NAN : -INFINITY;
      free(S); free(phs); free(slot);
      continue;
    }
    double m = -INFINITY;
    for (int64_t t = 0; t < n; ++t) if (S[t] > m) m = S[t];
    double l = 0.0;
    for (int64_t t = 0; t < n; ++t) { S[t] = exp(S[t] - m); l += S[t]; }
    for (int64_t t = 0; t < n; ++t) {
      double p = S[t] / l;
      size_t vbase = ((((size_t)phs[t] * s->Hkv + g) * P) + slot[t]) * d;
      for (int i = 0; i < d; ++i) o[i] += p * ld(v_pool, s->dtype, vbase + i);
    }
    if (lse) lse[row] = m + log(l);
    free(S); free(phs); free(slot);
  }
}
