// abi.hip -- the C ABI of libentmaxkv.so (declared in include/entmaxkv.h):
// argument validation, workspace sizing and kernel launches.  Nothing here
// allocates device memory or synchronizes.
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "launch.hpp"

namespace ekv {

// --------------------------------------------------------- Gauss-Hermite rule
// Nodes: sign changes of the orthonormal Hermite polynomial p_16 on a fine grid,
// refined by bisection; weights: Christoffel numbers 1 / sum_{k<16} p_k(x)^2.
// (p_0 = pi^(-1/4), p_1 = sqrt(2) x p_0,
//  p_{k+1} = sqrt(2/(k+1)) x p_k - sqrt(k/(k+1)) p_{k-1}.)
static void ortho_hermite(double x, double *pk /*[17]*/) {
  pk[0] = std::pow(M_PI, -0.25);
  pk[1] = std::sqrt(2.0) * x * pk[0];
  for (int k = 1; k < 16; ++k)
    pk[k + 1] = std::sqrt(2.0 / (k + 1)) * x * pk[k] - std::sqrt((double)k / (k + 1)) * pk[k - 1];
}

static GaussConsts compute_gh16() {
  GaussConsts gc;
  double pk[17];
  int found = 0;
  const double step = 1e-3;
  double xa = -7.0;
  ortho_hermite(xa, pk);
  double fa = pk[16];
  for (int i = 1; i <= 14000 && found < 16; ++i) {
    const double xb = -7.0 + i * step;
    ortho_hermite(xb, pk);
    const double fb = pk[16];
    if ((fa < 0) != (fb < 0)) {
      double lo = xa, hi = xb, flo = fa;
      for (int it = 0; it < 200; ++it) {
        const double mid = 0.5 * (lo + hi);
        if (mid == lo || mid == hi) break;
        ortho_hermite(mid, pk);
        if ((pk[16] < 0) == (flo < 0)) { lo = mid; flo = pk[16]; } else hi = mid;
      }
      // pick the end with the smaller |p_16|
      double plo, phi;
      ortho_hermite(lo, pk); plo = std::fabs(pk[16]);
      ortho_hermite(hi, pk); phi = std::fabs(pk[16]);
      gc.x[found++] = plo <= phi ? lo : hi;
    }
    xa = xb;
    fa = fb;
  }
  for (int j = 0; j < 16; ++j) {
    ortho_hermite(gc.x[j], pk);
    double s = 0.0;
    for (int k = 0; k < 16; ++k) s += pk[k] * pk[k];
    gc.w[j] = (1.0 / s) / std::sqrt(M_PI);  // normalized: sum_j w_j = 1
  }
  return gc;
}

const GaussConsts &gauss_consts() {
  static const GaussConsts gc = compute_gh16();
  return gc;
}

static thread_local char g_err[256] = "";

static int32_t hip_status(hipError_t e) {
  if (e == hipSuccess) return ENTMAXKV_OK;
  std::snprintf(g_err, sizeof g_err, "HIP error: %s", hipGetErrorString(e));
  return ENTMAXKV_ERR_HIP;
}

static int32_t check_shape(const entmaxkv_shape *s, Dims *D) {
  if (!s) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (s->batch < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1 || s->max_pages < 1 ||
      s->num_phys_pages < 1 || s->head_dim < 1 || s->page_size < 1)
    return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (s->n_q_heads % s->n_kv_heads != 0) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (!(s->scale >= 0.0) || !std::isfinite(s->scale)) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (s->dtype != ENTMAXKV_F32 && s->dtype != ENTMAXKV_BF16) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  const int G = s->n_q_heads / s->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return ENTMAXKV_ERR_UNSUPPORTED;
  if (s->head_dim != 64 && s->head_dim != 128) return ENTMAXKV_ERR_UNSUPPORTED;
  if (s->page_size != 16 && s->page_size != 32 && s->page_size != 64) return ENTMAXKV_ERR_UNSUPPORTED;
  if ((long long)s->batch * s->n_q_heads > 8192) return ENTMAXKV_ERR_UNSUPPORTED;
  if ((long long)s->max_pages * s->page_size >= (1ll << 31) || s->max_pages >= (1 << 24))
    return ENTMAXKV_ERR_UNSUPPORTED;
  if ((long long)s->num_phys_pages * s->n_kv_heads * s->page_size >= (1ll << 32)) return ENTMAXKV_ERR_UNSUPPORTED;
  if (D) {
    D->B = s->batch;
    D->Hq = s->n_q_heads;
    D->Hkv = s->n_kv_heads;
    D->G = G;
    D->d = s->head_dim;
    D->P = s->page_size;
    D->max_pages = s->max_pages;
    D->num_phys = s->num_phys_pages;
    D->scale = s->scale != 0.0 ? s->scale : 1.0 / std::sqrt((double)s->head_dim);
  }
  return ENTMAXKV_OK;
}

static int32_t check_ws(size_t need, const void *ws, size_t ws_bytes) {
  if (need == 0) return ENTMAXKV_OK;
  if (!ws || ws_bytes < need) return ENTMAXKV_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  return ENTMAXKV_OK;
}

static bool misaligned16(const void *a, const void *b = nullptr, const void *c = nullptr) {
  return ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) | reinterpret_cast<uintptr_t>(c)) & 15) != 0;
}

}  // namespace ekv

using namespace ekv;

// ---------------------------------------------------------------- measurement probe
// Reads a buffer with coalesced 16-byte loads (eight in flight per thread) and
// keeps the loads alive through a checksum that is stored only if it equals a
// fixed value: the HBM read rate of a plain stream on this GPU.
namespace {
typedef unsigned int probe_u32x4 __attribute__((ext_vector_type(4)));
constexpr int kProbeUnroll = 8;
__global__ __launch_bounds__(256) void stream_read_kernel(const probe_u32x4 *__restrict__ src, size_t n16,
                                                          uint32_t *__restrict__ sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * 256 * kProbeUnroll;
  for (size_t base = (size_t)blockIdx.x * 256 * kProbeUnroll + threadIdx.x; base < n16; base += stride) {
    probe_u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const size_t i = base + (size_t)u * 256;
      v[u] = src[i < n16 ? i : n16 - 1];
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}
}  // namespace

// score_select_pages_gauss: the scorer's table, the bracket summary, the selector's workspace
static size_t score_gauss_ws_bytes(const Dims &D) {
  Carve cv(nullptr);
  cv.take<char>(score_ws_bytes(D));
  cv.take<double>(score_summary_doubles(D));
  cv.take<char>(gauss_ws_bytes(D));
  return cv.bytes();
}

extern "C" {

size_t entmaxkv_workspace_bytes(const entmaxkv_shape *shape, int32_t which_call) {
  Dims D;
  if (check_shape(shape, &D) != ENTMAXKV_OK) return 0;
  switch (which_call) {
    case ENTMAXKV_CALL_SCORE: return score_ws_bytes(D);
    case ENTMAXKV_CALL_TOPK: return topk_ws_bytes(D);
    case ENTMAXKV_CALL_GAUSS: return gauss_ws_bytes(D);
    case ENTMAXKV_CALL_DECODE_SPARSE: return decode_ws_bytes(D, false);
    case ENTMAXKV_CALL_DECODE_FULL: return full_ws_bytes(D);
    case ENTMAXKV_CALL_SOFTMAX: return softmax_ws_bytes(D);
    case ENTMAXKV_CALL_SOFTMAX_SPARSE: return softmax_sparse_ws_bytes(D);
    case ENTMAXKV_CALL_TOPK_GROUP: return topk_group_ws_bytes(D);
    case ENTMAXKV_CALL_GAUSS_GROUP: return gauss_group_ws_bytes(D);
    case ENTMAXKV_CALL_DECODE_GROUP: return decode_group_ws_bytes(D);
    case ENTMAXKV_CALL_SCORE_GAUSS: return score_gauss_ws_bytes(D);
  }
  return 0;
}

size_t entmaxkv_decode_workspace_bytes(const entmaxkv_shape *shape, int32_t which_call, int64_t max_kept_pages) {
  Dims D;
  if (check_shape(shape, &D) != ENTMAXKV_OK) return 0;
  if (which_call != ENTMAXKV_CALL_DECODE_SPARSE && which_call != ENTMAXKV_CALL_DECODE_GROUP &&
      which_call != ENTMAXKV_CALL_DECODE_FULL)
    return 0;
  if (max_kept_pages < 0) return 0;
  return decode_ws_bytes_items(D, (long long)max_kept_pages);
}

const char *entmaxkv_status_string(int32_t status) {
  switch (status) {
    case ENTMAXKV_OK: return "ok";
    case ENTMAXKV_ERR_INVALID_ARGUMENT: return "invalid argument";
    case ENTMAXKV_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case ENTMAXKV_ERR_WORKSPACE: return "workspace missing or too small";
    case ENTMAXKV_ERR_HIP: return g_err[0] ? g_err : "HIP error";
    case ENTMAXKV_ERR_TOO_LARGE: return "shape needs more than the library's static scratch holds";
  }
  return "unknown status";
}

void entmaxkv_gauss_hermite16(double *nodes, double *weights) {
  const GaussConsts &gc = gauss_consts();
  for (int j = 0; j < 16; ++j) {
    if (nodes) nodes[j] = gc.x[j];
    if (weights) weights[j] = gc.w[j] * std::sqrt(M_PI);
  }
}

int32_t build_page_meta(const entmaxkv_shape *shape, const void *k_pool, const int32_t *page_table,
                        const int32_t *seq_lens, const int32_t *from_token, void *meta,
                        hipStream_t stream) {
  Dims D;
  int32_t st = check_shape(shape, &D);
  if (st) return st;
  if (!k_pool || !page_table || !seq_lens || !meta) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (misaligned16(k_pool, meta)) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  return hip_status(launch_build_meta(D, shape->dtype, false, k_pool, page_table, seq_lens, from_token, meta, stream));
}

int32_t build_page_meta_f8(const entmaxkv_shape *shape, const void *k_pool, const int32_t *page_table,
                           const int32_t *seq_lens, const int32_t *from_token, void *meta,
                           hipStream_t stream) {
  Dims D;
  int32_t st = check_shape(shape, &D);
  if (st) return st;
  if (shape->dtype != ENTMAXKV_BF16) return ENTMAXKV_ERR_UNSUPPORTED;
  if (!k_pool || !page_table || !seq_lens || !meta) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (misaligned16(k_pool, meta)) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  return hip_status(launch_build_meta(D, shape->dtype, true, k_pool, page_table, seq_lens, from_token, meta, stream));
}

int32_t append_token(const entmaxkv_shape *shape, const void *k_new, const void *v_new, void *k_pool,
                     void *v_pool, const int32_t *page_table, const int32_t *seq_lens, void *meta,
                     int32_t meta_format, hipStream_t stream) {
  Dims D;
  int32_t st = check_shape(shape, &D);
  if (st) return st;
  if (!k_new || !v_new || !k_pool || !v_pool || !page_table || !seq_lens || !meta)
    return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (meta_format != 0 && meta_format != 1) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (meta_format == 1 && shape->dtype != ENTMAXKV_BF16) return ENTMAXKV_ERR_UNSUPPORTED;
  return hip_status(launch_append_token(D, shape->dtype, meta_format == 1, k_new, v_new, k_pool, v_pool, page_table,
                                        seq_lens, meta, stream));
}

int32_t score_pages(const entmaxkv_shape *shape, const void *q, const void *meta,
                    const int32_t *page_table, const int32_t *seq_lens, float *box, float *mu,
                    float *var, void *ws, size_t ws_bytes, hipStream_t stream) {
  Dims D;
  int32_t st = check_shape(shape, &D);
  if (st) return st;
  if (!q || !meta || !page_table || !seq_lens || !box || !mu || !var) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (misaligned16(q, meta)) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if ((st = check_ws(score_ws_bytes(D), ws, ws_bytes))) return st;
  return hip_status(launch_score(D, shape->dtype, false, q, meta, page_table, seq_lens, box, mu, var, ws, stream));
}

int32_t score_pages_noalloc(const entmaxkv_shape *shape, const void *q, const void *meta,
                            const int32_t *page_table, const int32_t *seq_lens, float *box, float *mu,
                            float *var, hipStream_t stream) {
  Dims D;
  int32_t st = check_shape(shape, &D);
  if (st) return st;
  if (!q || !meta || !page_table || !seq_lens || !box || !mu || !var) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (misaligned16(q, meta)) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (score_ws_bytes(D) > score_scratch_bytes()) return ENTMAXKV_ERR_TOO_LARGE;
  return hip_status(launch_score_noalloc(D, shape->dtype, q, meta, page_table, seq_lens, box, mu, var, stream));
}

size_t entmaxkv_score_scratch_bytes(void) { return score_scratch_bytes(); }

int32_t score_pages_f8(const entmaxkv_shape *shape, const void *q, const void *meta,
                       const int32_t *page_table, const int32_t *seq_lens, float *box, float *mu,
                       float *var, void *ws, size_t ws_bytes, hipStream_t stream) {
  Dims D;
  int32_t st = check_shape(shape, &D);
  if (st) return st;
  if (shape->dtype != ENTMAXKV_BF16) return ENTMAXKV_ERR_UNSUPPORTED;
  if (!q || !meta || !page_table || !seq_lens || !box || !mu || !var) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (misaligned16(q, meta)) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if ((st = check_ws(score_ws_bytes(D), ws, ws_bytes))) return st;
  return hip_status(launch_score(D, shape->dtype, true, q, meta, page_table, seq_lens, box, mu, var, ws, stream));
}

int32_t select_pages_topk(const entmaxkv_shape *shape, const float *box, const int32_t *seq_lens,
                          int32_t k, const uint8_t *seq_mask, int32_t *sel_idx, int32_t *sel_cnt,
                          void *ws, size_t ws_bytes, hipStream_t stream) {
  Dims D;
  int32_t st = check_shape(shape, &D);
  if (st) return st;
  if (!box || !seq_lens || !sel_idx || !sel_cnt || k <= 0) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if ((st = check_ws(topk_ws_bytes(D), ws, ws_bytes))) return st;
  return hip_status(launch_topk(D, box, seq_lens, k, seq_mask, sel_idx, sel_cnt, ws, stream));
}

int32_t score_select_pages_gauss(const entmaxkv_shape *shape, const void *q, const void *meta,
                                 const int32_t *page_table, const int32_t *seq_lens, float *box, float *mu,
                                 float *var, double alpha, double delta, double n_sigma, const uint8_t *seq_mask,
                                 int32_t *sel_idx, int32_t *sel_cnt, double *tau_hat, void *ws, size_t ws_bytes,
                                 hipStream_t stream) {
  Dims D;
  int32_t st = check_shape(shape, &D);
  if (st) return st;
  if (!q || !meta || !page_table || !seq_lens || !box || !mu || !var || !sel_idx || !sel_cnt)
    return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (misaligned16(q, meta)) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (!(alpha > 1.0) || !std::isfinite(alpha) || !(delta >= 0.0) || !std::isfinite(delta) ||
      !(n_sigma >= 0.0) || !std::isfinite(n_sigma))
    return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if ((st = check_ws(score_gauss_ws_bytes(D), ws, ws_bytes))) return st;
  Carve cv(ws);
  void *ws_score = cv.take<char>(score_ws_bytes(D));
  double *summ = cv.take<double>(score_summary_doubles(D));
  void *ws_gauss = cv.take<char>(gauss_ws_bytes(D));
  ScoreSummary sm;
  sm.summ = summ;
  sm.x_top = gauss_consts().x[15];
  sm.nzero = gauss_zero_words(D, ws_gauss, &sm.zero);
  hipError_t e = launch_score_summary(D, shape->dtype, q, meta, page_table, seq_lens, box, mu, var, ws_score, sm,
                                      stream);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(launch_gauss_from_summary(D, box, mu, var, seq_lens, alpha, delta, n_sigma, seq_mask, sel_idx,
                                              sel_cnt, tau_hat, summ, ws_gauss, stream));
}

int32_t select_pages_gauss(const entmaxkv_shape *shape, const float *box, const float *mu,
                           const float *var, const int32_t *seq_lens, double alpha, double delta,
                           double n_sigma, const uint8_t *seq_mask, int32_t *sel_idx,
                           int32_t *sel_cnt, double *tau_hat, void *ws, size_t ws_bytes,
                           hipStream_t stream) {
  Dims D;
  int32_t st = check_shape(shape, &D);
  if (st) return st;
  if (!box || !mu || !var || !seq_lens || !sel_idx || !sel_cnt) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (!(alpha > 1.0) || !std::isfinite(alpha) || !(delta >= 0.0) || !std::isfinite(delta) ||
      !(n_sigma >= 0.0) || !std::isfinite(n_sigma))
    return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if ((st = check_ws(gauss_ws_bytes(D), ws, ws_bytes))) return st;
  return hip_status(launch_gauss(D, box, mu, var, seq_lens, alpha, delta, n_sigma, seq_mask, sel_idx,
                                 sel_cnt, tau_hat, ws, stream));
}

static int32_t decode_common(const entmaxkv_shape *shape, const void *q, const void *k_pool,
                             const void *v_pool, const int32_t *page_table, const int32_t *seq_lens,
                             const int32_t *sel_idx, const int32_t *sel_cnt, double alpha,
                             int32_t tau_method, float *out, double *tau, float *weights_out, void *ws,
                             size_t ws_bytes, hipStream_t stream, bool full) {
  Dims D;
  int32_t st = check_shape(shape, &D);
  if (st) return st;
  if (!q || !k_pool || !v_pool || !page_table || !seq_lens || !out) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (misaligned16(q, k_pool, v_pool)) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (!full && (!sel_idx || !sel_cnt)) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (!(alpha > 1.0) || !std::isfinite(alpha)) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (tau_method != 0 && tau_method != 1) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (tau_method == 1 && alpha != 2.0) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if ((st = check_ws(decode_ws_min_bytes(D), ws, ws_bytes))) return st;
  if (full)
    return hip_status(launch_entmax_full(D, shape->dtype, q, k_pool, v_pool, page_table, seq_lens, alpha,
                                         tau_method, out, tau, weights_out, ws, ws_bytes, stream));
  return hip_status(launch_entmax_decode(D, shape->dtype, q, k_pool, v_pool, page_table, seq_lens, sel_idx,
                                         sel_cnt, alpha, tau_method, out, tau, weights_out, ws, ws_bytes, stream));
}

int32_t entmax_decode_sparse(const entmaxkv_shape *shape, const void *q, const void *k_pool,
                             const void *v_pool, const int32_t *page_table,
                             const int32_t *seq_lens, const int32_t *sel_idx,
                             const int32_t *sel_cnt, double alpha, int32_t tau_method, float *out,
                             double *tau, float *weights_out, void *ws, size_t ws_bytes,
                             hipStream_t stream) {
  return decode_common(shape, q, k_pool, v_pool, page_table, seq_lens, sel_idx, sel_cnt, alpha,
                       tau_method, out, tau, weights_out, ws, ws_bytes, stream, false);
}

int32_t select_pages_topk_group(const entmaxkv_shape *shape, const float *box, const int32_t *seq_lens,
                                int32_t k, const uint8_t *seq_mask, int32_t *sel_idx, int32_t *sel_cnt,
                                void *ws, size_t ws_bytes, hipStream_t stream) {
  Dims D;
  int32_t st = check_shape(shape, &D);
  if (st) return st;
  if (!box || !seq_lens || !sel_idx || !sel_cnt || k <= 0) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if ((st = check_ws(topk_group_ws_bytes(D), ws, ws_bytes))) return st;
  return hip_status(launch_topk_group(D, box, seq_lens, k, seq_mask, sel_idx, sel_cnt, ws, stream));
}

int32_t select_pages_gauss_group(const entmaxkv_shape *shape, const float *box, const float *mu,
                                 const float *var, const int32_t *seq_lens, double alpha, double delta,
                                 double n_sigma, const uint8_t *seq_mask, int32_t *sel_idx,
                                 int32_t *sel_cnt, double *tau_hat, void *ws, size_t ws_bytes,
                                 hipStream_t stream) {
  Dims D;
  int32_t st = check_shape(shape, &D);
  if (st) return st;
  if (!box || !mu || !var || !seq_lens || !sel_idx || !sel_cnt) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (!(alpha > 1.0) || !std::isfinite(alpha) || !(delta >= 0.0) || !std::isfinite(delta) ||
      !(n_sigma >= 0.0) || !std::isfinite(n_sigma))
    return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if ((st = check_ws(gauss_group_ws_bytes(D), ws, ws_bytes))) return st;
  return hip_status(launch_gauss_group(D, box, mu, var, seq_lens, alpha, delta, n_sigma, seq_mask, sel_idx,
                                       sel_cnt, tau_hat, ws, stream));
}

int32_t entmax_decode_sparse_group(const entmaxkv_shape *shape, const void *q, const void *k_pool,
                                   const void *v_pool, const int32_t *page_table, const int32_t *seq_lens,
                                   const int32_t *sel_idx, const int32_t *sel_cnt, double alpha,
                                   int32_t tau_method, float *out, double *tau, float *weights_out, void *ws,
                                   size_t ws_bytes, hipStream_t stream) {
  Dims D;
  int32_t st = check_shape(shape, &D);
  if (st) return st;
  if (!q || !k_pool || !v_pool || !page_table || !seq_lens || !out || !sel_idx || !sel_cnt)
    return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (misaligned16(q, k_pool, v_pool)) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (!(alpha > 1.0) || !std::isfinite(alpha)) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (tau_method != 0 && tau_method != 1) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (tau_method == 1 && alpha != 2.0) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if ((st = check_ws(decode_ws_min_bytes(D), ws, ws_bytes))) return st;
  return hip_status(launch_entmax_decode_group(D, shape->dtype, q, k_pool, v_pool, page_table, seq_lens, sel_idx,
                                               sel_cnt, alpha, tau_method, out, tau, weights_out, ws, ws_bytes,
                                               stream));
}

int32_t entmax_decode_full(const entmaxkv_shape *shape, const void *q, const void *k_pool,
                           const void *v_pool, const int32_t *page_table, const int32_t *seq_lens,
                           double alpha, int32_t tau_method, float *out, double *tau,
                           float *weights_out, void *ws, size_t ws_bytes, hipStream_t stream) {
  return decode_common(shape, q, k_pool, v_pool, page_table, seq_lens, nullptr, nullptr, alpha,
                       tau_method, out, tau, weights_out, ws, ws_bytes, stream, true);
}

int32_t softmax_decode_full(const entmaxkv_shape *shape, const void *q, const void *k_pool,
                            const void *v_pool, const int32_t *page_table,
                            const int32_t *seq_lens, float *out, float *lse, void *ws,
                            size_t ws_bytes, hipStream_t stream) {
  Dims D;
  int32_t st = check_shape(shape, &D);
  if (st) return st;
  if (!q || !k_pool || !v_pool || !page_table || !seq_lens || !out) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (misaligned16(q, k_pool, v_pool)) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if ((st = check_ws(softmax_ws_bytes(D), ws, ws_bytes))) return st;
  return hip_status(launch_softmax(D, shape->dtype, q, k_pool, v_pool, page_table, seq_lens, out, lse, ws, stream));
}

int32_t softmax_decode_sparse(const entmaxkv_shape *shape, const void *q, const void *k_pool,
                              const void *v_pool, const int32_t *page_table,
                              const int32_t *seq_lens, const int32_t *sel_idx,
                              const int32_t *sel_cnt, float *out, float *lse, void *ws,
                              size_t ws_bytes, hipStream_t stream) {
  Dims D;
  int32_t st = check_shape(shape, &D);
  if (st) return st;
  if (!q || !k_pool || !v_pool || !page_table || !seq_lens || !sel_idx || !sel_cnt || !out)
    return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if (misaligned16(q, k_pool, v_pool)) return ENTMAXKV_ERR_INVALID_ARGUMENT;
  if ((st = check_ws(softmax_sparse_ws_bytes(D), ws, ws_bytes))) return st;
  return hip_status(launch_softmax_sparse(D, shape->dtype, q, k_pool, v_pool, page_table, seq_lens, sel_idx,
                                          sel_cnt, out, lse, ws, stream));
}

int32_t entmaxkv_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15) != 0)
    return ENTMAXKV_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL(stream_read_kernel, dim3(1024), dim3(256), 0, stream,
                     reinterpret_cast<const probe_u32x4 *>(src), bytes / 16, sink);
  return hip_status(hipGetLastError());
}

}  // extern "C"

