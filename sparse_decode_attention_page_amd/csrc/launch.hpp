// launch.hpp -- host-side launchers of the EntmaxKV kernels (internal to the
// library; the public C ABI is include/entmaxkv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.hpp"

namespace ekv {

// workspace carving helper: every region 256-byte aligned
struct Carve {
  char *base;
  size_t off;
  explicit Carve(void *p) : base(static_cast<char *>(p)), off(0) {}
  template <typename T>
  T *take(size_t count) {
    off = (off + 255) & ~(size_t)255;
    T *p = base ? reinterpret_cast<T *>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
  size_t bytes() const { return (off + 255) & ~(size_t)255; }
};

struct GaussConsts {
  double x[16];  // Gauss-Hermite nodes, ascending
  double w[16];  // weights divided by sqrt(pi)
};
const GaussConsts &gauss_consts();

hipError_t launch_build_meta(const Dims &D, int dtype, bool f8, const void *k_pool, const int32_t *page_table,
                             const int32_t *seq_lens, const int32_t *from_token, void *meta,
                             hipStream_t s);

hipError_t launch_append_token(const Dims &D, int dtype, bool f8, const void *k_new, const void *v_new, void *k_pool,
                               void *v_pool, const int32_t *page_table, const int32_t *seq_lens, void *meta,
                               hipStream_t s);

size_t score_ws_bytes(const Dims &D);
hipError_t launch_score(const Dims &D, int dtype, bool f8, const void *q, const void *meta,
                        const int32_t *page_table, const int32_t *seq_lens, float *box, float *mu,
                        float *var, void *ws, hipStream_t s);

// score_pages that also writes the Gaussian selector's bracket terms (two
// doubles per (query row, 64-page tile): the largest mean over the tile's valid
// full pages, the largest mu + sqrt2 sigma x_top over its valid pages) to summ,
// and zeroes the nzero words at zero (the selector's counts and counters).
constexpr int kSummaryTile = 64;  // pages per summary entry (the scorer's tile)
struct ScoreSummary {
  double *summ = nullptr;
  double x_top = 0.0;
  unsigned *zero = nullptr;
  long long nzero = 0;
};
size_t score_summary_doubles(const Dims &D);
hipError_t launch_score_summary(const Dims &D, int dtype, const void *q, const void *meta,
                                const int32_t *page_table, const int32_t *seq_lens, float *box, float *mu,
                                float *var, void *ws, const ScoreSummary &sm, hipStream_t s);

// score_pages with the coefficient table in the library's static device scratch
size_t score_scratch_bytes();
hipError_t launch_score_noalloc(const Dims &D, int dtype, const void *q, const void *meta,
                                const int32_t *page_table, const int32_t *seq_lens, float *box, float *mu,
                                float *var, hipStream_t s);

size_t topk_ws_bytes(const Dims &D);
hipError_t launch_topk(const Dims &D, const float *box, const int32_t *seq_lens, int k,
                       const uint8_t *seq_mask, int32_t *sel_idx, int32_t *sel_cnt, void *ws,
                       hipStream_t s);

size_t gauss_ws_bytes(const Dims &D);
hipError_t launch_gauss(const Dims &D, const float *box, const float *mu, const float *var,
                        const int32_t *seq_lens, double alpha, double delta, double n_sigma,
                        const uint8_t *seq_mask, int32_t *sel_idx, int32_t *sel_cnt,
                        double *tau_hat, void *ws, hipStream_t s);
// The selector's words that must be zero before its counting launch (counts
// and arrival counters, contiguous at the start of its workspace region
// returned in *zero), for a caller whose own launch zeroes them; then
// launch_gauss_from_summary runs the selector with the bracket read from the
// scorer's summary (summ, tiles_per_row entries per row) instead of its own
// bracket launch.
long long gauss_zero_words(const Dims &D, void *ws, unsigned **zero);
hipError_t launch_gauss_from_summary(const Dims &D, const float *box, const float *mu, const float *var,
                                     const int32_t *seq_lens, double alpha, double delta, double n_sigma,
                                     const uint8_t *seq_mask, int32_t *sel_idx, int32_t *sel_cnt,
                                     double *tau_hat, const double *summ, void *ws, hipStream_t s);

// Decode workspaces: the item capacity (kept pages over all query-head rows)
// follows from the bytes given; decode_ws_bytes is the size for every row's
// full set, decode_ws_bytes_items the size for `items` kept pages and
// decode_ws_min_bytes the size for one.
size_t decode_ws_bytes(const Dims &D, bool full);
size_t decode_ws_bytes_items(const Dims &D, long long items);
size_t decode_ws_min_bytes(const Dims &D);
hipError_t launch_entmax_decode(const Dims &D, int dtype, const void *q, const void *k_pool,
                                const void *v_pool, const int32_t *page_table,
                                const int32_t *seq_lens, const int32_t *sel_idx,
                                const int32_t *sel_cnt, double alpha, int tau_method, float *out,
                                double *tau, float *weights_out, void *ws, size_t ws_bytes, hipStream_t s);

// per-item decode (a set per query head, few rows) into a workspace of `cap` items
size_t decode_items_ws_bytes(const Dims &D, long long cap);
hipError_t launch_entmax_decode_items(const Dims &D, int dtype, const void *q, const void *k_pool,
                                      const void *v_pool, const int32_t *page_table, const int32_t *seq_lens,
                                      const int32_t *sel_idx, const int32_t *sel_cnt, double alpha, int tau_method,
                                      float *out, double *tau, float *weights_out, void *ws, long long cap,
                                      hipStream_t s);

size_t decode_group_ws_bytes(const Dims &D);
hipError_t launch_entmax_decode_group(const Dims &D, int dtype, const void *q, const void *k_pool,
                                      const void *v_pool, const int32_t *page_table, const int32_t *seq_lens,
                                      const int32_t *sel_idx, const int32_t *sel_cnt, double alpha, int tau_method,
                                      float *out, double *tau, float *weights_out, void *ws, size_t ws_bytes,
                                      hipStream_t s);

size_t topk_group_ws_bytes(const Dims &D);
hipError_t launch_topk_group(const Dims &D, const float *box, const int32_t *seq_lens, int k,
                             const uint8_t *seq_mask, int32_t *sel_idx, int32_t *sel_cnt, void *ws,
                             hipStream_t s);
size_t gauss_group_ws_bytes(const Dims &D);
hipError_t launch_gauss_group(const Dims &D, const float *box, const float *mu, const float *var,
                              const int32_t *seq_lens, double alpha, double delta, double n_sigma,
                              const uint8_t *seq_mask, int32_t *sel_idx, int32_t *sel_cnt, double *tau_hat,
                              void *ws, hipStream_t s);

size_t full_ws_bytes(const Dims &D);
hipError_t launch_entmax_full(const Dims &D, int dtype, const void *q, const void *k_pool, const void *v_pool,
                              const int32_t *page_table, const int32_t *seq_lens, double alpha, int tau_method,
                              float *out, double *tau, float *weights_out, void *ws, size_t ws_bytes,
                              hipStream_t s);

size_t softmax_ws_bytes(const Dims &D);
size_t softmax_sparse_ws_bytes(const Dims &D);
hipError_t launch_softmax_sparse(const Dims &D, int dtype, const void *q, const void *k_pool, const void *v_pool,
                                 const int32_t *page_table, const int32_t *seq_lens, const int32_t *sel_idx,
                                 const int32_t *sel_cnt, float *out, float *lse, void *ws, hipStream_t s);
hipError_t launch_softmax(const Dims &D, int dtype, const void *q, const void *k_pool,
                          const void *v_pool, const int32_t *page_table, const int32_t *seq_lens,
                          float *out, float *lse, void *ws, hipStream_t s);

}  // namespace ekv
