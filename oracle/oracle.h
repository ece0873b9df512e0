/*
 * oracle.h -- plain, slow fp64 CPU reference for the EntmaxKV decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library) never calls it and shares no code with it.
 *
 * Source being followed ("the EntmaxKV summary" below):
 *   "Resumen Tecnico: EntmaxKV - Decodificacion Consciente del Soporte para
 *   Atencion Entmax", gist.science/es/paper/2605.21649 (with its ja/ko/ar
 *   translations), sections 2.A (query-aware page scoring), 2.B (selection
 *   policies), 2.C (sparse entmax attention) and 3 (theory).
 * The summary prints no formula for alpha-entmax; the definition used is the
 * standard one of Peters, Niculae & Martins (2019), "Sparse Sequence-to-
 * Sequence Models": p_t = [(alpha-1) s_t - tau]_+^(1/(alpha-1)), sum p = 1.
 *
 * Layouts (row-major, element types given by `dtype`: 0 = fp32, 1 = bf16):
 *   q        [B][Hq][d]
 *   k, v     [num_phys][Hkv][P][d]
 *   meta     [num_phys][Hkv][4][d]     (k_min, k_max, mean, var)
 *   page_table int32 [B][max_pages],   seq_lens int32 [B]
 *   per-page outputs  [B][Hq][max_pages],  per-token weights [B][Hq][max_pages*P]
 * Query head h reads KV head h / (Hq/Hkv).
 */
#ifndef ENTMAXKV_ORACLE_H
#define ENTMAXKV_ORACLE_H
#include <stdint.h>

typedef struct {
  int32_t B, Hq, Hkv, d, P, max_pages, num_phys, dtype;
  double scale; /* score scale c_d; 0 selects 1/sqrt(d) */
} orc_shape;

/* storage roundings used at the interface */
double orc_round_bf16(double x);   /* round-to-nearest-even to bfloat16 */
double orc_round_f32(double x);    /* round-to-nearest-even to float32 */
double orc_round_f32_up(double x); /* round toward +infinity to float32 */
/* OCP FP8 E4M3 (no infinities, NaN = 0x7F/0xFF, largest finite 448): exact
 * decode; encode = nearest, ties to even, saturating at +-448. */
double orc_e4m3_decode(uint8_t c);
uint8_t orc_e4m3_encode(double x);

/* 16-point Gauss-Hermite rule (weight exp(-x^2)) by Golub-Welsch. */
void orc_gauss_hermite16(double *nodes, double *weights);

void orc_build_page_meta(const orc_shape *s, const void *k_pool, const int32_t *page_table,
                         const int32_t *seq_lens, const int32_t *from_token, void *meta);
/* compact records for bf16 keys: [num_phys][Hkv] of
 * k_min bf16[d] | k_max bf16[d] | mean e4m3[d] | var e4m3[d]  (6d bytes) */
void orc_build_page_meta_f8(const orc_shape *s, const void *k_pool, const int32_t *page_table,
                            const int32_t *seq_lens, const int32_t *from_token, void *meta);

/* rows: optional list of (b*Hq+h) rows to compute (NULL = all).  Outputs are
 * float32 arrays; entries of rows not listed and pages >= N_b are untouched. */
void orc_score_pages(const orc_shape *s, const void *q, const void *meta,
                     const int32_t *page_table, const int32_t *seq_lens,
                     const int32_t *rows, int32_t n_rows,
                     float *box, float *mu, float *var);
/* the same scores from compact records */
void orc_score_pages_f8(const orc_shape *s, const void *q, const void *meta,
                        const int32_t *page_table, const int32_t *seq_lens,
                        const int32_t *rows, int32_t n_rows,
                        float *box, float *mu, float *var);

void orc_select_topk(const orc_shape *s, const float *box, const int32_t *seq_lens, int32_t k,
                     const uint8_t *seq_mask, const int32_t *rows, int32_t n_rows,
                     int32_t *sel_idx, int32_t *sel_cnt);

void orc_select_gauss(const orc_shape *s, const float *box, const float *mu, const float *var,
                      const int32_t *seq_lens, double alpha, double delta, double n_sigma,
                      const uint8_t *seq_mask, const int32_t *rows, int32_t n_rows,
                      int32_t *sel_idx, int32_t *sel_cnt, double *tau_hat);

/* Group-shared selection (one set per KV head; rows = group rows b*Hkv+g):
 * Top-k on the largest box over the G heads; Gaussian = union of the G heads'
 * sets.  sel_idx [B][Hkv][max_pages], sel_cnt [B][Hkv], tau_hat [B][Hq]. */
void orc_select_topk_group(const orc_shape *s, const float *box, const int32_t *seq_lens, int32_t k,
                           const uint8_t *seq_mask, const int32_t *rows, int32_t n_rows,
                           int32_t *sel_idx, int32_t *sel_cnt);
void orc_select_gauss_group(const orc_shape *s, const float *box, const float *mu, const float *var,
                            const int32_t *seq_lens, double alpha, double delta, double n_sigma,
                            const uint8_t *seq_mask, const int32_t *rows, int32_t n_rows,
                            int32_t *sel_idx, int32_t *sel_cnt, double *tau_hat);

/* F(tau) of the Gaussian selector over an explicit page list (for pins). */
double orc_gauss_mass(const float *mu, const float *var, const int32_t *n, int32_t np, double alpha,
                      double tau);

/* sel_idx == NULL: every page of the sequence is kept (full-cache decode). */
void orc_entmax_decode(const orc_shape *s, const void *q, const void *k_pool, const void *v_pool,
                       const int32_t *page_table, const int32_t *seq_lens,
                       const int32_t *sel_idx, const int32_t *sel_cnt, double alpha,
                       const int32_t *rows, int32_t n_rows,
                       double *out, double *tau, double *weights);

void orc_softmax_decode(const orc_shape *s, const void *q, const void *k_pool, const void *v_pool,
                        const int32_t *page_table, const int32_t *seq_lens,
                        const int32_t *sel_idx, const int32_t *sel_cnt,
                        const int32_t *rows, int32_t n_rows, double *out, double *lse);

/* alpha-entmax threshold of one score vector by bisection (exposed for pins). */
double orc_entmax_tau(const double *scores, int64_t n, double alpha);

#endif
