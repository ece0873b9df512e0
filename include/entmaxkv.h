/*
 * entmaxkv.h -- C ABI of libentmaxkv.so, the EntmaxKV decode hot path for one
 * AMD Instinct MI355X (gfx950), written as HIP kernels.
 *
 * What it computes follows "Resumen Tecnico: EntmaxKV - Decodificacion
 * Consciente del Soporte para Atencion Entmax" (gist.science/es/paper/
 * 2605.21649; cited below as [EntmaxKV s.X] for its section X):
 *   1. per-page key metadata: per-coordinate bounding box and Gaussian
 *      statistics ............................................ [EntmaxKV s.2.A]
 *   2. query-aware page scores from that metadata ............. [EntmaxKV s.2.A]
 *   3. candidate-page selection, Top-k or Gaussian-aware ...... [EntmaxKV s.2.B]
 *   4. alpha-entmax attention over the selected pages only .... [EntmaxKV s.2.C]
 *   plus full-cache entmax and softmax decodes, the baselines of [EntmaxKV s.4].
 * alpha-entmax is p_t = [(alpha-1) s_t - tau]_+^(1/(alpha-1)) with tau fixed by
 * sum_t p_t = 1 (Peters, Niculae & Martins 2019); scores s_t = scale * q.k_t.
 *
 * Conventions shared by every call
 * --------------------------------
 *  * Pointers are DEVICE pointers unless marked (host).  The caller owns every
 *    buffer, including the workspace `ws`; the library allocates nothing, keeps
 *    no pointer after returning and holds no state between calls (apart from
 *    lazily computed constants), so calls on different streams may overlap as
 *    long as their buffers (including `ws`) do not.
 *  * All work is enqueued asynchronously on `stream`; nothing synchronizes.
 *    Launch failures are reported by the return code; device faults surface at
 *    the caller's next synchronization.
 *  * Arguments are validated on the host before anything is launched.  Device
 *    data (page ids, lengths, selections) is checked inside the kernels, which
 *    never read outside the buffers implied by the shape; bad entries produce
 *    NaN results as documented per call.
 *  * q, k_pool, v_pool and meta must be 16-byte aligned (vector loads);
 *    a misaligned pointer is rejected with ENTMAXKV_ERR_INVALID_ARGUMENT.
 *  * KV dtype (`entmaxkv_shape.dtype`) applies to q, the K/V pools and the page
 *    metadata; outputs are float32 (scores, weights, attention outputs) or
 *    float64 (thresholds).
 *
 * Layouts (row-major):
 *   q           [B][Hq][d]                       KV dtype
 *   k_pool,v_pool [num_phys_pages][Hkv][P][d]    KV dtype (slot j of a page = token p*P+j)
 *   meta        [num_phys_pages][Hkv][4][d]      KV dtype: k_min, k_max, mean, var
 *   page_table  int32 [B][max_pages]             logical page -> physical page
 *   seq_lens    int32 [B]                        L_b, clamped to [0, max_pages*P]
 *   box, mu, var  float32 [B][Hq][max_pages]     per-page scores
 *   sel_idx     int32 [B][Hq][max_pages]         selected logical pages, strictly ascending
 *   sel_cnt     int32 [B][Hq]
 *   out         float32 [B][Hq][d]
 * Query head h reads KV head h / (Hq/Hkv).  Logical page p of sequence b holds
 * n_{b,p} = min(P, L_b - p*P) tokens; N_b = ceil(L_b/P) pages.
 */
#ifndef ENTMAXKV_H
#define ENTMAXKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum entmaxkv_status {
  ENTMAXKV_OK = 0,
  ENTMAXKV_ERR_INVALID_ARGUMENT = 1, /* null required pointer, bad dims, Hq % Hkv, k <= 0, alpha <= 1, ... */
  ENTMAXKV_ERR_UNSUPPORTED = 2,      /* (d, P, dtype, group size) without a kernel */
  ENTMAXKV_ERR_WORKSPACE = 3,        /* ws_bytes below entmaxkv_workspace_bytes(...) */
  ENTMAXKV_ERR_HIP = 4,              /* a launch failed; see entmaxkv_status_string */
  ENTMAXKV_ERR_TOO_LARGE = 5         /* shape beyond score_pages_noalloc's static scratch */
};

enum entmaxkv_dtype { ENTMAXKV_F32 = 0, ENTMAXKV_BF16 = 1 };

/* Supported: d in {64, 128}; P in {16, 32, 64}; Hq/Hkv in {1, 2, 4, 8};
 * B*Hq <= 8192; max_pages*P < 2^31; num_phys_pages*Hkv*P < 2^32 (pool rows are
 * indexed in 32 bits).  Other shapes return ENTMAXKV_ERR_UNSUPPORTED. */
typedef struct entmaxkv_shape {
  int32_t batch;          /* B >= 1 */
  int32_t n_q_heads;      /* Hq >= 1 */
  int32_t n_kv_heads;     /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;       /* d */
  int32_t page_size;      /* P */
  int32_t max_pages;      /* >= 1; row stride of page_table and of per-page arrays */
  int32_t num_phys_pages; /* >= 1; size of the K/V/metadata pools */
  int32_t dtype;          /* entmaxkv_dtype */
  double scale;           /* score scale; 0 selects 1/sqrt(d) */
} entmaxkv_shape;

/* which_call values for entmaxkv_workspace_bytes */
enum entmaxkv_call {
  ENTMAXKV_CALL_SCORE = 1,
  ENTMAXKV_CALL_TOPK = 2,
  ENTMAXKV_CALL_GAUSS = 3,
  ENTMAXKV_CALL_DECODE_SPARSE = 4,
  ENTMAXKV_CALL_DECODE_FULL = 5,
  ENTMAXKV_CALL_SOFTMAX = 6,
  ENTMAXKV_CALL_SOFTMAX_SPARSE = 7,
  ENTMAXKV_CALL_TOPK_GROUP = 8,
  ENTMAXKV_CALL_GAUSS_GROUP = 9,
  ENTMAXKV_CALL_DECODE_GROUP = 10,
  ENTMAXKV_CALL_SCORE_GAUSS = 11
};

/* Bytes of workspace a call needs for this shape (0 if none).  Returns 0 for
 * an invalid shape.  The workspace content need not be initialized and is
 * scratch: its contents after a call are unspecified. */
size_t entmaxkv_workspace_bytes(const entmaxkv_shape *shape /*(host)*/, int32_t which_call);

/* Decode workspaces sized by a bound on the kept pages instead of the full
 * cache.  which_call: ENTMAXKV_CALL_DECODE_SPARSE, _GROUP or _FULL (0 for any
 * other call or a negative bound).  max_kept_pages bounds the kept pages
 * summed over all query-head rows (b, h): sum of sel_cnt for the per-head
 * call, G times the sum of the group counts for the group call, sum of N_b
 * times Hq for the full call.  entmaxkv_workspace_bytes gives the size for
 * every row's full set; any size from entmaxkv_decode_workspace_bytes(shape,
 * call, 1) up is accepted, and the workspace then holds the kept pages the
 * bytes allow: rows are laid out in row order, and a row whose pages end past
 * that capacity gets NaN out and tau (its weights_out row stays zero).  The
 * capacity for a workspace of B bytes is therefore the largest n with
 * entmaxkv_decode_workspace_bytes(shape, call, n) <= B. */
size_t entmaxkv_decode_workspace_bytes(const entmaxkv_shape *shape /*(host)*/, int32_t which_call,
                                       int64_t max_kept_pages);

/* Text for a status code; for ENTMAXKV_ERR_HIP it includes the HIP error of
 * the most recent failure on the calling thread. */
const char *entmaxkv_status_string(int32_t status);

/*
 * build_page_meta -- [EntmaxKV s.2.A]: per page and KV head, the per-coordinate
 * key bounding box (k_min, k_max) and Gaussian statistics (mean, population
 * variance) over the page's filled tokens.  mean = S1/n, var = max(0, S2/n -
 * mean^2) with S1, S2 fp64 sums; each value is rounded once (round-to-nearest-
 * even) to the KV dtype.  from_token (nullable): when given, only logical pages
 * p < N_b whose range [pP, pP+P) holds a position >= from_token[b] are rebuilt
 * (the append path as pages fill); NULL rebuilds every page.  Records of pages
 * whose page-table entry is out of range are left untouched.
 */
int32_t build_page_meta(const entmaxkv_shape *shape, const void *k_pool, const int32_t *page_table,
                        const int32_t *seq_lens, const int32_t *from_token, void *meta,
                        hipStream_t stream);

/*
 * score_pages -- [EntmaxKV s.2.A], per (b, h, p < N_b) with c = scale:
 *   box = c * sum_i max(q_i kmin_i, q_i kmax_i)   (upper bound on every score in
 *         the page; stored rounded toward +inf)
 *   mu  = c * sum_i q_i mean_i,   var = c^2 * sum_i q_i^2 var_i
 *         (Gaussian model of the page's scores; stored round-to-nearest-even)
 * Each sum is taken in fp64 over i = 0 .. d-1 in that order, adding each term
 * once (bf16 products and f32 products with q and k are exact in fp64; an f32
 * q_i^2 var_i is rounded to fp64 first), so the stored floats equal an fp64
 * evaluation of these definitions in index order bit for bit.  Keys are
 * assumed finite (an infinite k_min / k_max may give a NaN box).
 * Entries p >= N_b are not written.  An out-of-range page-table entry gives NaN
 * in all three outputs.  ws: entmaxkv_workspace_bytes(shape, ENTMAXKV_CALL_SCORE).
 */
int32_t score_pages(const entmaxkv_shape *shape, const void *q, const void *meta,
                    const int32_t *page_table, const int32_t *seq_lens, float *box, float *mu,
                    float *var, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * score_pages_noalloc -- score_pages for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): same arguments, outputs and rules as score_pages, but no
 * workspace argument.  Its scratch (the query coefficient table, 32 B * batch *
 * n_q_heads * head_dim) is a static device array of
 * entmaxkv_score_scratch_bytes() = 4 MiB inside the library, one per GPU, kept
 * until the process ends; a shape needing more returns ENTMAXKV_ERR_TOO_LARGE
 * before anything is launched (batch * n_q_heads * head_dim <= 131072 fits).
 * The call allocates nothing.  Every call on one GPU uses that GPU's array, so
 * calls that overlap on one GPU (different streams, or other host threads)
 * race; serialize them.  Nothing in the scratch has to start at zero.
 */
int32_t score_pages_noalloc(const entmaxkv_shape *shape, const void *q, const void *meta,
                            const int32_t *page_table, const int32_t *seq_lens, float *box, float *mu,
                            float *var, hipStream_t stream);
size_t entmaxkv_score_scratch_bytes(void);

/*
 * append_token -- the streaming side of [EntmaxKV s.2.A]: the page metadata
 * is kept current as pages fill.  For every sequence b with L_b = seq_lens[b]
 * >= 1 (seq_lens already count the new token; L_b is clamped to
 * max_pages * P as in every call): the new token's key and value rows
 * k_new / v_new [B][Hkv][d] (KV dtype) are written to slot (L_b - 1) % P of
 * logical page (L_b - 1) / P in k_pool / v_pool, and that page's metadata
 * record is rebuilt over its filled slots by the code build_page_meta (or
 * build_page_meta_f8 when meta_format = 1; bf16 keys only) runs, in the same
 * order of additions, so it equals a rebuild of the page bit for bit.  A
 * sequence whose page-table entry is out of range is left untouched.  One
 * launch; no workspace.
 */
int32_t append_token(const entmaxkv_shape *shape, const void *k_new, const void *v_new, void *k_pool,
                     void *v_pool, const int32_t *page_table, const int32_t *seq_lens, void *meta,
                     int32_t meta_format, hipStream_t stream);

/*
 * Compact metadata -- the records above with the Gaussian moments stored in
 * 8 bits, a variant the summary leaves open ([EntmaxKV s.2.A] only asks for
 * "lightweight" per-page statistics).  bf16 keys only (ENTMAXKV_ERR_UNSUPPORTED
 * otherwise).  Record [num_phys][Hkv] of 6d bytes:
 *   k_min bf16[d] | k_max bf16[d] | mean e4m3[d] | var e4m3[d]
 * e4m3 = OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities; 0x7F / 0xFF are NaN; largest finite value 448).
 * build_page_meta_f8: k_min / k_max exactly as build_page_meta; mean and var
 * (fp64, as there) rounded to the nearest E4M3 value, ties to even, magnitudes
 * >= 448 saturating to +-448.  from_token as in build_page_meta.
 * score_pages_f8: score_pages over compact records, with the same outputs,
 * fp64 sums of exact products and roundings (a NaN code gives NaN mu / var);
 * ws: entmaxkv_workspace_bytes(shape, ENTMAXKV_CALL_SCORE).
 * meta must be 16-byte aligned; 6d is a multiple of 16 for d in {64, 128}.
 */
int32_t build_page_meta_f8(const entmaxkv_shape *shape, const void *k_pool,
                           const int32_t *page_table, const int32_t *seq_lens,
                           const int32_t *from_token, void *meta, hipStream_t stream);
int32_t score_pages_f8(const entmaxkv_shape *shape, const void *q, const void *meta,
                       const int32_t *page_table, const int32_t *seq_lens, float *box, float *mu,
                       float *var, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * select_pages_topk -- [EntmaxKV s.2.B, policy 1]: per (b, h), the k pages with
 * the largest box; ties go to the lower page index, NaN ranks below every
 * number, -0 equals +0, and N_b <= k keeps every page.  sel_idx lists the
 * chosen pages in ascending order, sel_cnt = min(k, N_b).  seq_mask (nullable,
 * uint8 [B]): rows of sequences with mask 0 are not written.
 */
int32_t select_pages_topk(const entmaxkv_shape *shape, const float *box, const int32_t *seq_lens,
                          int32_t k, const uint8_t *seq_mask, int32_t *sel_idx, int32_t *sel_cnt,
                          void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * select_pages_gauss -- [EntmaxKV s.2.B, policy 2]: estimate the global entmax
 * threshold from the page Gaussians, then keep pages whose estimated maximum
 * score reaches it minus a margin Delta.  This library's reading:
 *   F(t) = sum_p n_p sum_j w_j [(alpha-1)(mu_p + sqrt(2) sigma_p x_j) - t]_+^(1/(alpha-1))
 * with (x_j, w_j sqrt(pi)) the 16-point Gauss-Hermite rule; tau_hat is the root
 * of F = 1; keep p iff min(mu_p + n_sigma*sigma_p, box_p) >= tau_hat/(alpha-1)
 * - delta; if none passes, keep the page of largest estimate (lowest index on
 * ties).  Pages with non-finite box/mu/var are never kept.  tau_hat (nullable,
 * float64 [B][Hq]) receives tau_hat/(alpha-1) (score units); NaN if N_b = 0.
 * Requires alpha > 1, delta >= 0, n_sigma >= 0.  alpha in {1.5, 2} runs the
 * chunked solver (integer counts to locate the root, then an exact solve on a
 * window of them); other alpha use a slower per-row bisection.  The result is
 * deterministic: the same inputs give the same tau_hat bits and sets on every
 * call (every sum is an integer add or taken in a fixed order).
 * ws: entmaxkv_workspace_bytes(shape, ENTMAXKV_CALL_GAUSS).
 */
int32_t select_pages_gauss(const entmaxkv_shape *shape, const float *box, const float *mu,
                           const float *var, const int32_t *seq_lens, double alpha, double delta,
                           double n_sigma, const uint8_t *seq_mask, int32_t *sel_idx,
                           int32_t *sel_cnt, double *tau_hat, void *ws, size_t ws_bytes,
                           hipStream_t stream);

/*
 * score_select_pages_gauss -- score_pages followed by select_pages_gauss in one
 * call ([EntmaxKV s.2.A] then [s.2.B, policy 2]): the same box/mu/var,
 * sel_idx/sel_cnt and tau_hat bits as the two calls made in turn (same
 * arguments, same meaning, same errors), with the selector's bracket (the
 * largest lone-page bound and the largest top quadrature point of each row)
 * taken from maxima the scoring launch writes as it stores mu and var, so the
 * selector's own pass over the statistics for it is not run.  bf16 or fp32
 * records (not the compact format).  Both steps are asynchronous on `stream`.
 * ws: entmaxkv_workspace_bytes(shape, ENTMAXKV_CALL_SCORE_GAUSS).
 */
int32_t score_select_pages_gauss(const entmaxkv_shape *shape, const void *q, const void *meta,
                                 const int32_t *page_table, const int32_t *seq_lens, float *box, float *mu,
                                 float *var, double alpha, double delta, double n_sigma, const uint8_t *seq_mask,
                                 int32_t *sel_idx, int32_t *sel_cnt, double *tau_hat, void *ws, size_t ws_bytes,
                                 hipStream_t stream);

/*
 * entmax_decode_sparse -- [EntmaxKV s.2.C]: alpha-entmax attention of each
 * query head over the tokens t < L_b of ITS selected pages only:
 *   p_t = [(alpha-1) s_t - tau]_+^(1/(alpha-1)) / Z,  out = sum_t p_t v_t,
 * tau the root of sum_t [(alpha-1)s_t - tau]_+^(1/(alpha-1)) = 1 over the kept
 * tokens, Z the sum of the unnormalized weights.  tau_method: 0 = root finder
 * (any alpha), 1 = sparsemax sort closed form (alpha == 2 only; any other
 * alpha with tau_method 1 is ENTMAXKV_ERR_INVALID_ARGUMENT).  The sort runs
 * over the row's candidate tokens, those above a certified lower bound on tau
 * (every other token is outside the support), when at most 1024 of them
 * remain and the row keeps at most 4096 tokens above its slices' first cut;
 * any other row is solved by the root finder, which reaches the same tau to
 * fp64 resolution.  tau (nullable, float64 [B][Hq]) receives tau/(alpha-1).
 * weights_out (nullable, float32 [B][Hq][max_pages*P], for tests) receives p
 * at logical token positions and zero elsewhere.  A row with sel_cnt = 0 gets
 * out = 0, tau = NaN; a row whose selection is out of range or not strictly
 * ascending gets NaN out and tau.  The heads of a KV group are scored
 * together: each page kept by any of them is read once per KV head.  Results
 * are identical from run to run (every sum has a fixed order).
 * ws: entmaxkv_workspace_bytes(shape, ENTMAXKV_CALL_DECODE_SPARSE), or a
 * kept-page-bounded size from entmaxkv_decode_workspace_bytes.
 */
int32_t entmax_decode_sparse(const entmaxkv_shape *shape, const void *q, const void *k_pool,
                             const void *v_pool, const int32_t *page_table,
                             const int32_t *seq_lens, const int32_t *sel_idx,
                             const int32_t *sel_cnt, double alpha, int32_t tau_method, float *out,
                             double *tau, float *weights_out, void *ws, size_t ws_bytes,
                             hipStream_t stream);

/*
 * Group-shared selection -- one kept set per KV head, for the G = Hq/Hkv query
 * heads that read it, so the decode fetches each kept page once.  The policies
 * of [EntmaxKV s.2.B] are stated per query; this grouping is a variant the
 * summary leaves open.  Group sets: sel_idx int32 [B][Hkv][max_pages]
 * (ascending), sel_cnt int32 [B][Hkv].
 * select_pages_topk_group: per (b, g), the k pages with the largest
 *   max_h box[b][g G + h][p] over the group's heads (a NaN box ranks below
 *   every number; ties to the lower page; N_b <= k keeps every page).
 *   ws: entmaxkv_workspace_bytes(shape, ENTMAXKV_CALL_TOPK_GROUP).
 * select_pages_gauss_group: per (b, g), the union of the G heads' sets as
 *   select_pages_gauss computes them (page p kept iff some head h keeps it:
 *   the largest margin est_{h,p} - (tau_hat_h/(alpha-1) - Delta) is >= 0, or p
 *   is a head's fallback page).  tau_hat (nullable) [B][Hq] as there.
 *   ws: entmaxkv_workspace_bytes(shape, ENTMAXKV_CALL_GAUSS_GROUP).
 * entmax_decode_sparse_group: entmax_decode_sparse with every head h of KV
 *   head g attending over the group's set sel_idx[b][g]; outputs, tau,
 *   weights_out, malformed-selection rules and tau_method as there (a
 *   malformed group set makes all G rows NaN).  Each kept K page is read once
 *   per group.  ws: entmaxkv_workspace_bytes(shape, ENTMAXKV_CALL_DECODE_GROUP)
 *   or a kept-page-bounded size (entmaxkv_decode_workspace_bytes).
 * seq_mask (nullable, uint8 [B]): as in the per-head calls.
 */
int32_t select_pages_topk_group(const entmaxkv_shape *shape, const float *box, const int32_t *seq_lens,
                                int32_t k, const uint8_t *seq_mask, int32_t *sel_idx, int32_t *sel_cnt,
                                void *ws, size_t ws_bytes, hipStream_t stream);
int32_t select_pages_gauss_group(const entmaxkv_shape *shape, const float *box, const float *mu,
                                 const float *var, const int32_t *seq_lens, double alpha, double delta,
                                 double n_sigma, const uint8_t *seq_mask, int32_t *sel_idx,
                                 int32_t *sel_cnt, double *tau_hat, void *ws, size_t ws_bytes,
                                 hipStream_t stream);
int32_t entmax_decode_sparse_group(const entmaxkv_shape *shape, const void *q, const void *k_pool,
                                   const void *v_pool, const int32_t *page_table, const int32_t *seq_lens,
                                   const int32_t *sel_idx, const int32_t *sel_cnt, double alpha,
                                   int32_t tau_method, float *out, double *tau, float *weights_out, void *ws,
                                   size_t ws_bytes, hipStream_t stream);

/* entmax_decode_full -- the same attention over every cached token (the
 * full-cache entmax baseline of [EntmaxKV s.4]).  tau_method, tau,
 * weights_out and the alpha rules as in entmax_decode_sparse (the sort form
 * runs over the candidates of the whole cache under the same 1024 limit).
 * ws: entmaxkv_workspace_bytes(shape, ENTMAXKV_CALL_DECODE_FULL). */
int32_t entmax_decode_full(const entmaxkv_shape *shape, const void *q, const void *k_pool,
                           const void *v_pool, const int32_t *page_table, const int32_t *seq_lens,
                           double alpha, int32_t tau_method, float *out, double *tau,
                           float *weights_out, void *ws, size_t ws_bytes, hipStream_t stream);

/* softmax_decode_full -- exact softmax attention over every cached token, the
 * full-cache softmax baseline of [EntmaxKV s.4].  lse (nullable, float32
 * [B][Hq]) receives log sum_t exp(s_t).  L_b = 0 gives out = 0, lse = -inf. */
int32_t softmax_decode_full(const entmaxkv_shape *shape, const void *q, const void *k_pool,
                            const void *v_pool, const int32_t *page_table,
                            const int32_t *seq_lens, float *out, float *lse, void *ws,
                            size_t ws_bytes, hipStream_t stream);

/*
 * softmax_decode_sparse -- softmax attention over the kept pages only: the
 * comparison of [EntmaxKV s.3] (under one kept set, softmax gives weight to
 * every discarded token, so its discarded mass is positive, while entmax loses
 * nothing once the kept set contains its support) and [EntmaxKV s.4]
 * (discarded mass and relative output error, entmax vs softmax sparse decoding
 * at equal KV budgets).  Selection contract as entmax_decode_sparse: per query
 * row, sel_cnt in [0, N_b] and sel_idx[0 .. sel_cnt) ascending logical pages
 * < N_b; a violation or an out-of-range page-table entry gives NaN in out and
 * lse.  out: float32 [B][Hq][d] = sum_{t in T} softmax_T(s)_t v_t over the kept
 * tokens T (t < L_b); lse (nullable, float32 [B][Hq]): log sum_{t in T} exp(s_t),
 * -inf with out = 0 when T is empty.  fp32 arithmetic (as softmax_decode_full).
 * ws: entmaxkv_workspace_bytes(shape, ENTMAXKV_CALL_SOFTMAX_SPARSE).
 */
int32_t softmax_decode_sparse(const entmaxkv_shape *shape, const void *q, const void *k_pool,
                              const void *v_pool, const int32_t *page_table,
                              const int32_t *seq_lens, const int32_t *sel_idx,
                              const int32_t *sel_cnt, float *out, float *lse, void *ws,
                              size_t ws_bytes, hipStream_t stream);

/* The 16-point Gauss-Hermite rule the Gaussian selector uses (host copy, for
 * inspection): nodes ascending, weights for the weight function exp(-x^2). */
/* Measurement probe, not part of the decode path: reads `bytes` of device memory
 * at src (16-byte aligned, bytes a multiple of 16) with coalesced 16-byte loads
 * and no other traffic (one 4-byte store to sink only if a checksum matches a
 * fixed value), so that its duration gives the HBM read rate this GPU sustains.
 * Returns ENTMAXKV_OK or ENTMAXKV_ERR_INVALID_ARGUMENT / ENTMAXKV_ERR_HIP. */
int32_t entmaxkv_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream);
void entmaxkv_gauss_hermite16(double *nodes /*(host)[16]*/, double *weights /*(host)[16]*/);

#ifdef __cplusplus
}
#endif
#endif
