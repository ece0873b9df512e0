// decode.hip -- alpha-entmax attention over selected pages ([EntmaxKV s.2.C]) and
// over the whole cache (the full-cache entmax baseline of [EntmaxKV s.4]).
//
// EntmaxKV s.2.C = section 2.C ("sparse entmax attention") of "Resumen Tecnico:
// EntmaxKV - Decodificacion Consciente del Soporte para Atencion Entmax",
// gist.science/es/paper/2605.21649: load only the KV entries of the selected
// pages and compute the alpha-entmax weights over that reduced set; when the
// selection contains the whole support the result is exact.
//
// alpha-entmax (Peters, Niculae & Martins 2019): with X_t = (alpha-1) s_t,
// p_t = [X_t - tau]_+^(1/(alpha-1)), tau the root of sum_t p_t = 1.
//
// Work is a flat list of items (row, i): the i-th selected page of query row
// (b, h).  Every block maps items through a prefix sum of the selection counts
// it computes itself, so no host round trip or extra launch is needed.
//  D1  per item: exact fp64 scores of the page's tokens into the workspace.
//      The last item of a row (atomic handshake) solves tau for the row:
//      safeguarded Newton from the left (F is convex and decreasing for
//      alpha <= 2), or the sparsemax sort closed form when asked for.
//  D2  per item: weighted sum of the page's V rows for the tokens above tau
//      (pages without such tokens read no V at all); the last item of a row
//      adds the per-page partials in page order.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace ekv {

constexpr int kDThreads = 256;
constexpr int kDGrid = 1024;   // persistent-style grid; items are strided over it
constexpr int kSortMax = 8192; // largest kept-token count sorted in LDS (alpha = 2)

struct DecodeWs {
  double *xs;          // [rows][max_pages*P]  X_t of kept tokens (item-major), -inf in empty slots
  float *part;         // [rows][max_pages][d] per-item partial outputs
  int *part_flag;      // [rows][max_pages]    1 if the item's partial is non-zero
  double *rowst;       // [rows][4]            tau (X units), Z, bad flag (0/1), unused
  unsigned long long *badf; // [rows]          == epoch when an item of the row is malformed
  unsigned long long *ctr;  // [rows][2]       epoch-tagged arrival counters (D1, D2)
  unsigned long long epoch;
};

struct DecodeParams {
  double a, beta, c;
  int ibeta, tau_method, full;
};

__device__ __forceinline__ double entw(double x, const DecodeParams &dp) {
  return dp.ibeta == 2 ? x * x : (dp.ibeta == 1 ? x : pow(x, dp.beta));
}
__device__ __forceinline__ double entw_d(double x, const DecodeParams &dp) {  // d/dx of entw
  return dp.ibeta == 2 ? 2.0 * x : (dp.ibeta == 1 ? 1.0 : dp.beta * pow(x, dp.beta - 1.0));
}

// Row item counts: selected pages (sparse) or all pages (full).  Returns the
// count clamped to [0, max_pages]; *bad set for malformed counts.
__device__ __forceinline__ int row_items(const Dims &D, const DecodeParams &dp, const int32_t *seq_lens,
                                         const int32_t *sel_cnt, int row, bool *bad) {
  const int b = row / D.Hq;
  const int np = n_pages_of(seq_len_clamped(seq_lens, b, D), D.P);
  *bad = false;
  if (dp.full) return np;
  int c = sel_cnt[row];
  if (c < 0 || c > np) { *bad = true; c = c < 0 ? 0 : (c > D.max_pages ? D.max_pages : c); }
  return c;
}

// Block-shared item map: prefix[r] = first item of row r.
__device__ void build_item_map(const Dims &D, const DecodeParams &dp, const int32_t *seq_lens,
                               const int32_t *sel_cnt, int *prefix, int rows, int *total) {
  __shared__ int scan_scratch[kDThreads / kWave];
  int run = 0;
  for (int r0 = 0; r0 < rows; r0 += kDThreads) {
    const int r = r0 + threadIdx.x;
    bool bad;
    const int c = r < rows ? row_items(D, dp, seq_lens, sel_cnt, r, &bad) : 0;
    int tot;
    const int ex = block_excl_scan(c, scan_scratch, &tot);
    if (r < rows) prefix[r] = run + ex;
    run += tot;
  }
  if (threadIdx.x == 0) prefix[rows] = run;
  __syncthreads();
  *total = run;
}
__device__ __forceinline__ int find_row(const int *prefix, int rows, int item) {
  int lo = 0, hi = rows - 1;  // largest r with prefix[r] <= item
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= item) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ------------------------------------------------------------ tau of one row
// Safeguarded Newton/bisection on F(t) = sum_t [X_t - t]_+^beta = 1 (all threads
// of the block call it; X in global memory, n entries, -inf entries ignored).
__device__ double solve_tau_block(const double *X, int n, const DecodeParams &dp, double *dred) {
  double mx = -INFINITY;
  int cnt = 0;
  for (int i = threadIdx.x; i < n; i += kDThreads) {
    const double x = X[i];
    if (x > -INFINITY) { mx = fmax(mx, x); ++cnt; }
  }
  mx = block_max(mx, dred);
  const double cntd = block_sum((double)cnt, dred);
  double lo = mx - 1.0;                              // F(lo) >= 1
  double hi = mx - pow(cntd, -dp.a);                 // F(hi) <= 1
  if (!(hi > lo)) return lo;
  double t = lo;
  bool bisect_next = false;
  for (int it = 0; it < 400; ++it) {
    double cand;
    if (bisect_next) {
      cand = 0.5 * (lo + hi);
    } else {
      double f = 0.0, fp = 0.0;
      for (int i = threadIdx.x; i < n; i += kDThreads) {
        const double x = X[i] - lo;
        if (x > 0.0) { f += entw(x, dp); fp += entw_d(x, dp); }
      }
      f = block_sum(f, dred);
      fp = block_sum(fp, dred);
      cand = fp > 0.0 ? lo + (f - 1.0) / fp : 0.5 * (lo + hi);
      if (!(cand > lo) || !(cand < hi)) {
        if (!(cand > lo) && f >= 1.0) break;  // Newton makes no progress: converged
        cand = 0.5 * (lo + hi);
      }
    }
    if (cand == lo || cand == hi) break;
    double f = 0.0;
    for (int i = threadIdx.x; i < n; i += kDThreads) {
      const double x = X[i] - cand;
      if (x > 0.0) f += entw(x, dp);
    }
    f = block_sum(f, dred);
    if (f >= 1.0) { lo = cand; bisect_next = false; }
    else { hi = cand; bisect_next = true; }
  }
  t = lo;
  return t;
}

// sparsemax closed form by a bitonic sort in LDS (n <= kSortMax)
__device__ double sparsemax_tau_sort(const double *X, int n, double *buf, int *scan_scratch) {
  int m = 1;
  while (m < n) m <<= 1;
  for (int i = threadIdx.x; i < m; i += kDThreads) buf[i] = i < n ? X[i] : -INFINITY;
  __syncthreads();
  for (int kk = 2; kk <= m; kk <<= 1) {  // sort descending
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < m; i += kDThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const bool desc = (i & kk) == 0;
          const double a = buf[i], b = buf[ixj];
          if (desc ? (a < b) : (a > b)) { buf[i] = b; buf[ixj] = a; }
        }
      }
      __syncthreads();
    }
  }
  // k* = max{k : 1 + k z_(k) > sum_{j<=k} z_(j)}; tau = (sum_{j<=k*} z_(j) - 1)/k*.
  // The condition holds exactly for k <= k*, so k* counts the k where it holds.
  // Prefix sums run chunk by chunk (wave scans + a carried running sum).
  __shared__ double wsum[kDThreads / kWave];
  __shared__ double s_sum;
  __shared__ int s_kstar;
  if (threadIdx.x == 0) { s_kstar = 0; s_sum = 0.0; }
  __syncthreads();
  double carry = 0.0;
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  for (int c0 = 0; c0 < n; c0 += kDThreads) {
    const int k = c0 + threadIdx.x;  // 0-based rank
    const double z = k < n ? buf[k] : 0.0;
    double x = z;
    for (int o = 1; o < kWave; o <<= 1) {
      const double y = __shfl_up(x, o, kWave);
      if (lane >= o) x += y;
    }
    if (lane == kWave - 1) wsum[wv] = x;
    __syncthreads();
    double off = carry;
    double tot = 0.0;
    for (int i = 0; i < kDThreads / kWave; ++i) {
      if (i < wv) off += wsum[i];
      tot += wsum[i];
    }
    const double cs = off + x;
    if (k < n && 1.0 + (double)(k + 1) * z > cs) {
      atomicMax(&s_kstar, k + 1);
    }
    __syncthreads();
    carry += tot;
  }
  // sum of the top k* values
  const int ks = s_kstar > 0 ? s_kstar : 1;
  double part = 0.0;
  for (int k = threadIdx.x; k < ks; k += kDThreads) part += buf[k];
  part = block_sum(part, wsum);
  (void)scan_scratch;
  return (part - 1.0) / (double)ks;
}

// --------------------------------------------------------------- D1: scores
template <typename T, int DIM>
__global__ __launch_bounds__(kDThreads) void decode_scores_kernel(
    Dims D, DecodeParams dp, const T *__restrict__ q, const T *__restrict__ k_pool,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ sel_idx, const int32_t *__restrict__ sel_cnt, float *__restrict__ out,
    double *__restrict__ tau_out, float *__restrict__ weights_out, DecodeWs ws) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ double dred[kDThreads / kWave];
  __shared__ double qs[DIM];
  __shared__ int s_last;
  const int rows = D.B * D.Hq;
  int *prefix = reinterpret_cast<int *>(smem);
  double *sortbuf = reinterpret_cast<double *>(smem + (((rows + 1) * 4 + 15) & ~15));
  int total;
  build_item_map(D, dp, seq_lens, sel_cnt, prefix, rows, &total);

  // rows without items: defined results now (no last block will come)
  for (int r = blockIdx.x; r < rows; r += gridDim.x) {
    bool bad;
    const int c = row_items(D, dp, seq_lens, sel_cnt, r, &bad);
    if (c == 0 && threadIdx.x == 0) {
      ws.rowst[r * 4 + 0] = NAN;
      ws.rowst[r * 4 + 1] = bad ? NAN : 0.0;
      ws.rowst[r * 4 + 2] = bad ? 1.0 : 0.0;
      if (tau_out) tau_out[r] = NAN;
    }
    if (c == 0) {
      for (int i = threadIdx.x; i < D.d; i += kDThreads) out[(size_t)r * D.d + i] = bad ? NAN : 0.0f;
    }
  }
  if (weights_out) {
    const size_t nw = (size_t)rows * D.max_pages * D.P;
    for (size_t i = (size_t)blockIdx.x * kDThreads + threadIdx.x; i < nw; i += (size_t)gridDim.x * kDThreads)
      weights_out[i] = 0.0f;
  }

  const int P = D.P;
  const int parts = kDThreads / P;          // threads per token
  const int per = DIM / parts;              // coordinates per thread
  const int tok = threadIdx.x / parts, part = threadIdx.x % parts;
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int r = find_row(prefix, rows, item);
    const int i = item - prefix[r];
    const int b = r / D.Hq, h = r % D.Hq, g = h / D.G;
    const int L = seq_len_clamped(seq_lens, b, D);
    const int np = n_pages_of(L, P);
    bool bad_item = false;
    int p = i;
    if (!dp.full) {
      p = sel_idx[(size_t)r * D.max_pages + i];
      if (p < 0 || p >= np) bad_item = true;
      else if (i > 0 && sel_idx[(size_t)r * D.max_pages + i - 1] >= p) bad_item = true;
    }
    int phys = -1;
    if (!bad_item) {
      phys = page_table[(size_t)b * D.max_pages + p];
      if (phys < 0 || phys >= D.num_phys) bad_item = true;
    }
    bool row_bad;
    const int cnt = row_items(D, dp, seq_lens, sel_cnt, r, &row_bad);
    double *xrow = ws.xs + (size_t)r * D.max_pages * P;
    __syncthreads();
    for (int t = threadIdx.x; t < DIM; t += kDThreads) qs[t] = (double)load_f<T>(q, (size_t)r * DIM + t);
    __syncthreads();
    if (bad_item) {
      if (threadIdx.x == 0) ws.badf[r] = ws.epoch;  // benign race: every writer stores the epoch
      for (int j = threadIdx.x; j < P; j += kDThreads) xrow[(size_t)i * P + j] = -INFINITY;
    } else {
      const int n = min(P, L - p * P);
      const T *kp = k_pool + (((size_t)phys * D.Hkv + g) * P + tok) * DIM + part * per;
      double acc = 0.0;
      if (tok < n) {
#pragma unroll 8
        for (int e = 0; e < per; ++e) acc += (double)load_f<T>(kp, e) * qs[part * per + e];
      }
      for (int o = parts / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, kWave);
      if (part == 0) xrow[(size_t)i * P + tok] = tok < n ? dp.a * (dp.c * acc) : -INFINITY;
    }
    if (!arrive_last_ep(&ws.ctr[r * 2 + 0], ws.epoch, (unsigned)cnt, &s_last)) continue;

    // ---- last item of row r: tau and the normalizer
    const int nX = cnt * P;
    double tau;
    if (dp.tau_method == 1 && dp.ibeta == 1 && nX <= kSortMax) tau = sparsemax_tau_sort(xrow, nX, sortbuf, nullptr);
    else tau = solve_tau_block(xrow, nX, dp, dred);
    double z = 0.0;
    for (int t = threadIdx.x; t < nX; t += kDThreads) {
      const double x = xrow[t] - tau;
      if (x > 0.0) z += entw(x, dp);
    }
    z = block_sum(z, dred);
    if (threadIdx.x == 0) {
      const bool badrow = row_bad || ws.badf[r] == ws.epoch;
      ws.rowst[r * 4 + 0] = tau;
      ws.rowst[r * 4 + 1] = z;
      ws.rowst[r * 4 + 2] = badrow ? 1.0 : 0.0;
      if (tau_out) tau_out[r] = badrow ? NAN : tau / dp.a;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------ D2: weighted V
template <typename T, int DIM>
__global__ __launch_bounds__(kDThreads) void decode_values_kernel(
    Dims D, DecodeParams dp, const T *__restrict__ v_pool, const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ sel_idx,
    const int32_t *__restrict__ sel_cnt, float *__restrict__ out, float *__restrict__ weights_out,
    DecodeWs ws) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float pw[64];
  __shared__ int s_last, s_any;
  __shared__ float red[kDThreads / (DIM / 2)][DIM];
  const int rows = D.B * D.Hq;
  int *prefix = reinterpret_cast<int *>(smem);
  int total;
  build_item_map(D, dp, seq_lens, sel_cnt, prefix, rows, &total);
  const int P = D.P;
  constexpr int kPairs = DIM / 2;
  const int cpair = threadIdx.x % kPairs, tg = threadIdx.x / kPairs;
  constexpr int TG = kDThreads / kPairs;
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int r = find_row(prefix, rows, item);
    const int i = item - prefix[r];
    const int b = r / D.Hq, h = r % D.Hq, g = h / D.G;
    bool row_bad;
    const int cnt = row_items(D, dp, seq_lens, sel_cnt, r, &row_bad);
    const double tau = ws.rowst[r * 4 + 0], z = ws.rowst[r * 4 + 1];
    const bool badrow = ws.rowst[r * 4 + 2] != 0.0;
    const double *xrow = ws.xs + (size_t)r * D.max_pages * P + (size_t)i * P;
    __syncthreads();
    if (threadIdx.x == 0) s_any = 0;
    __syncthreads();
    for (int j = threadIdx.x; j < P; j += kDThreads) {
      const double x = xrow[j] - tau;
      const float w = (x > 0.0) ? (float)(entw(x, dp) / z) : 0.0f;
      pw[j] = w;
      if (w != 0.0f) s_any = 1;
    }
    __syncthreads();
    const int L = seq_len_clamped(seq_lens, b, D);
    int p = dp.full ? i : sel_idx[(size_t)r * D.max_pages + i];
    const bool any = s_any != 0 && !badrow;
    if (weights_out && !badrow && p >= 0 && p < n_pages_of(L, P)) {
      for (int j = threadIdx.x; j < P; j += kDThreads)
        weights_out[(size_t)r * D.max_pages * P + (size_t)p * P + j] = pw[j];
    }
    if (any) {
      const int phys = page_table[(size_t)b * D.max_pages + p];
      const int n = min(P, L - p * P);
      const T *vp = v_pool + ((size_t)phys * D.Hkv + g) * (size_t)P * DIM;
      float a0 = 0.0f, a1 = 0.0f;
      for (int j = tg; j < n; j += TG) {
        const float wj = pw[j];
        if (wj == 0.0f) continue;
        float v0, v1;
        if constexpr (sizeof(T) == 2) {
          const uint32_t wv = reinterpret_cast<const uint32_t *>(vp + (size_t)j * DIM)[cpair];
          v0 = bf16lo(wv); v1 = bf16hi(wv);
        } else {
          const float2 wv = reinterpret_cast<const float2 *>(vp + (size_t)j * DIM)[cpair];
          v0 = wv.x; v1 = wv.y;
        }
        a0 += wj * v0;
        a1 += wj * v1;
      }
      red[tg][2 * cpair] = a0;
      red[tg][2 * cpair + 1] = a1;
      __syncthreads();
      for (int c2 = threadIdx.x; c2 < DIM; c2 += kDThreads) {
        float s = red[0][c2];
        for (int t = 1; t < TG; ++t) s += red[t][c2];
        ws.part[((size_t)r * D.max_pages + i) * DIM + c2] = s;
      }
    }
    if (threadIdx.x == 0) ws.part_flag[(size_t)r * D.max_pages + i] = any ? 1 : 0;
    if (!arrive_last_ep(&ws.ctr[r * 2 + 1], ws.epoch, (unsigned)cnt, &s_last)) continue;
    // ---- last item of row r: add the partials in page order
    for (int c2 = threadIdx.x; c2 < DIM; c2 += kDThreads) {
      float s = 0.0f;
      for (int t = 0; t < cnt; ++t)
        if (ws.part_flag[(size_t)r * D.max_pages + t]) s += ws.part[((size_t)r * D.max_pages + t) * DIM + c2];
      out[(size_t)r * DIM + c2] = badrow ? NAN : s;
    }
    __syncthreads();
  }
}

static DecodeWs carve_decode(const Dims &D, void *base, size_t *bytes) {
  Carve cv(base);
  const size_t rows = (size_t)D.B * D.Hq;
  DecodeWs w;
  w.xs = cv.take<double>(rows * D.max_pages * D.P);
  w.part = cv.take<float>(rows * D.max_pages * D.d);
  w.part_flag = cv.take<int>(rows * D.max_pages);
  w.rowst = cv.take<double>(rows * 4);
  w.badf = cv.take<unsigned long long>(rows);
  w.ctr = cv.take<unsigned long long>(rows * 2);
  w.epoch = 0;
  if (bytes) *bytes = cv.bytes();
  return w;
}

size_t decode_ws_bytes(const Dims &D, bool) {
  size_t b = 0;
  carve_decode(D, nullptr, &b);
  return b;
}

template <typename T, int DIM>
static hipError_t launch_decode_t(const Dims &D, const DecodeParams &dp, const void *q,
                                  const void *k_pool, const void *v_pool, const int32_t *page_table,
                                  const int32_t *seq_lens, const int32_t *sel_idx,
                                  const int32_t *sel_cnt, float *out, double *tau,
                                  float *weights_out, void *ws, hipStream_t s) {
  DecodeWs w = carve_decode(D, ws, nullptr);
  w.epoch = next_epoch();
  const int rows = D.B * D.Hq;
  const size_t map_bytes = (((size_t)(rows + 1) * 4 + 15) & ~(size_t)15);
  const size_t smem1 = map_bytes + (dp.tau_method == 1 ? (size_t)kSortMax * sizeof(double) : 0);
  const size_t smem2 = map_bytes;
  hipLaunchKernelGGL((decode_scores_kernel<T, DIM>), dim3(kDGrid), dim3(kDThreads), smem1, s, D, dp,
                     (const T *)q, (const T *)k_pool, page_table, seq_lens, sel_idx, sel_cnt, out, tau,
                     weights_out, w);
  hipLaunchKernelGGL((decode_values_kernel<T, DIM>), dim3(kDGrid), dim3(kDThreads), smem2, s, D, dp,
                     (const T *)v_pool, page_table, seq_lens, sel_idx, sel_cnt, out, weights_out, w);
  return hipGetLastError();
}

hipError_t launch_entmax_decode(const Dims &D, int dtype, const void *q, const void *k_pool,
                                const void *v_pool, const int32_t *page_table,
                                const int32_t *seq_lens, const int32_t *sel_idx,
                                const int32_t *sel_cnt, double alpha, int tau_method, float *out,
                                double *tau, float *weights_out, void *ws, hipStream_t s) {
  DecodeParams dp;
  dp.a = alpha - 1.0;
  dp.beta = 1.0 / dp.a;
  dp.c = D.scale;
  dp.ibeta = alpha == 1.5 ? 2 : (alpha == 2.0 ? 1 : 0);
  dp.tau_method = tau_method;
  dp.full = sel_idx == nullptr ? 1 : 0;
  if (dtype == ENTMAXKV_BF16) {
    if (D.d == 64) return launch_decode_t<uint16_t, 64>(D, dp, q, k_pool, v_pool, page_table, seq_lens, sel_idx, sel_cnt, out, tau, weights_out, ws, s);
    return launch_decode_t<uint16_t, 128>(D, dp, q, k_pool, v_pool, page_table, seq_lens, sel_idx, sel_cnt, out, tau, weights_out, ws, s);
  }
  if (D.d == 64) return launch_decode_t<float, 64>(D, dp, q, k_pool, v_pool, page_table, seq_lens, sel_idx, sel_cnt, out, tau, weights_out, ws, s);
  return launch_decode_t<float, 128>(D, dp, q, k_pool, v_pool, page_table, seq_lens, sel_idx, sel_cnt, out, tau, weights_out, ws, s);
}

}  // namespace ekv
