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

// per-launch epoch for arrival counters that may hold garbage (1 .. 2^40-1)
unsigned long long next_epoch();

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

size_t topk_ws_bytes(const Dims &D);
hipError_t launch_topk(const Dims &D, const float *box, const int32_t *seq_lens, int k,
                       const uint8_t *seq_mask, int32_t *sel_idx, int32_t *sel_cnt, void *ws,
                       hipStream_t s);

size_t gauss_ws_bytes(const Dims &D);
hipError_t launch_gauss(const Dims &D, const float *box, const float *mu, const float *var,
                        const int32_t *seq_lens, double alpha, double delta, double n_sigma,
                        const uint8_t *seq_mask, int32_t *sel_idx, int32_t *sel_cnt,
                        double *tau_hat, void *ws, hipStream_t s);

size_t decode_ws_bytes(const Dims &D, bool full);
hipError_t launch_entmax_decode(const Dims &D, int dtype, const void *q, const void *k_pool,
                                const void *v_pool, const int32_t *page_table,
                                const int32_t *seq_lens, const int32_t *sel_idx,
                                const int32_t *sel_cnt, double alpha, int tau_method, float *out,
                                double *tau, float *weights_out, void *ws, hipStream_t s);

size_t decode_group_ws_bytes(const Dims &D);
hipError_t launch_entmax_decode_group(const Dims &D, int dtype, const void *q, const void *k_pool,
                                      const void *v_pool, const int32_t *page_table, const int32_t *seq_lens,
                                      const int32_t *sel_idx, const int32_t *sel_cnt, double alpha, int tau_method,
                                      float *out, double *tau, float *weights_out, void *ws, hipStream_t s);

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
                              const int32_t *page_table, const int32_t *seq_lens, double alpha, float *out,
                              double *tau, float *weights_out, void *ws, hipStream_t s);

size_t softmax_ws_bytes(const Dims &D);
size_t softmax_sparse_ws_bytes(const Dims &D);
hipError_t launch_softmax_sparse(const Dims &D, int dtype, const void *q, const void *k_pool, const void *v_pool,
                                 const int32_t *page_table, const int32_t *seq_lens, const int32_t *sel_idx,
                                 const int32_t *sel_cnt, float *out, float *lse, void *ws, hipStream_t s);
hipError_t launch_softmax(const Dims &D, int dtype, const void *q, const void *k_pool,
                          const void *v_pool, const int32_t *page_table, const int32_t *seq_lens,
                          float *out, float *lse, void *ws, hipStream_t s);

}  // namespace ekv
