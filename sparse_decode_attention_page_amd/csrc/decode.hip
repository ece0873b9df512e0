// decode.hip -- alpha-entmax attention over selected pages ([EntmaxKV s.2.C]).
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
// One launch.  Work is a flat list of items (row, i): the i-th selected page of
// query row (b, h); every block maps items through a prefix sum of the
// selection counts it computes itself.
//  * item: exact fp64 scores of the page's tokens (bf16 products are exact;
//    fp64 sums), handed to the row's last block through the workspace;
//  * last item of a row (atomic handshake): stages the row's scores in LDS
//    with batched loads, solves tau by safeguarded Newton from
//    the left (F is convex and decreasing for alpha <= 2; bisection steps keep
//    it safe otherwise) or by the sparsemax sort closed form, then gathers the
//    V rows of the support tokens only and writes the output.  Kept tokens
//    outside the support cost no V traffic at all.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace ekv {

constexpr int kDThreads = 256;
constexpr int kDGrid = 1024;    // persistent-style grid; items are strided over it
constexpr int kStage = 4096;    // scores of a row staged in LDS by the last block
constexpr int kSortMax = 8192;  // largest kept-token count sorted in LDS (alpha = 2)
constexpr int kSupChunk = 1024; // support entries gathered per LDS pass

struct DecodeWs {
  double *xs;                // [rows][max_pages*P]  X_t of kept tokens (item-major), -inf in empty slots
  unsigned long long *badf;  // [rows]  == epoch when an item of the row is malformed
  unsigned long long *ctr;   // [rows]  epoch-tagged arrival counters
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

// Item count of a row: selected pages (sparse) or all pages (full), clamped to
// [0, max_pages]; *bad is set for a malformed count.
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

// Block-shared item map: prefix[r] = first item of row r, prefix[rows] = total.
__device__ int build_item_map(const Dims &D, const DecodeParams &dp, const int32_t *seq_lens,
                              const int32_t *sel_cnt, int *prefix, int rows, int *scan_scratch) {
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
  return run;
}
__device__ __forceinline__ int find_row(const int *prefix, int rows, int item) {
  int lo = 0, hi = rows - 1;  // largest r with prefix[r] <= item
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= item) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The scores of one row, as seen by the last block: the first kStage in LDS
// (staged once with batched loads), any remainder re-read from the workspace in
// batches.  Loops stay rolled: this code runs once per row and must stay small.
struct RowScores {
  double *xl;        // LDS copy of X[0 .. min(n, kStage))
  const double *X;   // the row in the workspace
  int n, ns;

  __device__ void load(const double *xrow, int nX, double *lds) {
    X = xrow;
    xl = lds;
    n = nX;
    ns = min(nX, kStage);
#pragma unroll 1
    for (int base = 0; base < ns; base += 8 * kDThreads) {
      double v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = ld_agent(&xrow[min(base + u * kDThreads + (int)threadIdx.x, ns - 1)]);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * kDThreads + threadIdx.x;
        if (i < ns) xl[i] = v[u];
      }
    }
    __syncthreads();
  }
  template <typename Fn>
  __device__ void for_each(Fn &&fn) const {
#pragma unroll 1
    for (int i = threadIdx.x; i < ns; i += kDThreads) fn(i, xl[i]);
#pragma unroll 1
    for (int base = ns; base < n; base += 8 * kDThreads) {
      double v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = ld_agent(&X[min(base + u * kDThreads + (int)threadIdx.x, n - 1)]);
#pragma unroll 1
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * kDThreads + threadIdx.x;
        if (i < n) fn(i, v[u]);
      }
    }
  }
  __device__ double at(int i) const { return i < ns ? xl[i] : ld_agent(&X[i]); }
};

// Root of F(t) = sum [X - t]_+^beta = 1: safeguarded Newton from the left.
__device__ __noinline__ double solve_tau(const RowScores &rs, const DecodeParams &dp, double *dred) {
  double mx = -INFINITY, cnt = 0.0;
  rs.for_each([&](int, double x) { if (x > -INFINITY) { mx = fmax(mx, x); cnt += 1.0; } });
  mx = block_max(mx, dred);
  cnt = block_sum(cnt, dred);
  double lo = mx - 1.0;               // F(lo) >= 1
  double hi = mx - pow(cnt, -dp.a);   // F(hi) <= 1
  if (!(hi > lo)) return lo;
  bool bisect_next = false;
#pragma unroll 1
  for (int it = 0; it < 400; ++it) {
    double cand;
    if (bisect_next) {
      cand = 0.5 * (lo + hi);
    } else {
      double f = 0.0, fp = 0.0;
      rs.for_each([&](int, double x) {
        const double y = x - lo;
        if (y > 0.0) { f += entw(y, dp); fp += entw_d(y, dp); }
      });
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
    rs.for_each([&](int, double x) {
      const double y = x - cand;
      if (y > 0.0) f += entw(y, dp);
    });
    f = block_sum(f, dred);
    if (f >= 1.0) { lo = cand; bisect_next = false; }
    else { hi = cand; bisect_next = true; }
  }
  return lo;
}

// sparsemax closed form (Martins & Astudillo 2016) by a bitonic sort in LDS:
// sort z descending; k* = max{k : 1 + k z_(k) > sum_{j<=k} z_(j)};
// tau = (sum_{j<=k*} z_(j) - 1) / k*.  The condition holds exactly for k <= k*.
__device__ double sparsemax_tau_sort(const RowScores &rs, double *buf, double *dred) {
  const int n = rs.n;
  int m = 1;
  while (m < n) m <<= 1;
  for (int i = threadIdx.x; i < m; i += kDThreads) buf[i] = i < n ? rs.at(i) : -INFINITY;
  __syncthreads();
  for (int kk = 2; kk <= m; kk <<= 1) {
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
  __shared__ double wsum[kDThreads / kWave];
  __shared__ int s_kstar;
  if (threadIdx.x == 0) s_kstar = 0;
  __syncthreads();
  double carry = 0.0;
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  for (int c0 = 0; c0 < n; c0 += kDThreads) {
    const int k = c0 + threadIdx.x;
    const double z = k < n ? buf[k] : 0.0;
    const bool finite = z > -INFINITY;
    double x = finite ? z : 0.0;
    for (int o = 1; o < kWave; o <<= 1) {
      const double y = __shfl_up(x, o, kWave);
      if (lane >= o) x += y;
    }
    if (lane == kWave - 1) wsum[wv] = x;
    __syncthreads();
    double off = carry, tot = 0.0;
    for (int i = 0; i < kDThreads / kWave; ++i) {
      if (i < wv) off += wsum[i];
      tot += wsum[i];
    }
    if (k < n && finite && 1.0 + (double)(k + 1) * z > off + x) atomicMax(&s_kstar, k + 1);
    __syncthreads();
    carry += tot;
  }
  const int ks = s_kstar > 0 ? s_kstar : 1;
  double part = 0.0;
  for (int k = threadIdx.x; k < ks; k += kDThreads) part += buf[k];
  part = block_sum(part, dred);
  return (part - 1.0) / (double)ks;
}

template <typename T, int DIM>
__global__ __launch_bounds__(kDThreads) void entmax_decode_kernel(
    Dims D, DecodeParams dp, const T *__restrict__ q, const T *__restrict__ k_pool,
    const T *__restrict__ v_pool, const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ sel_idx,
    const int32_t *__restrict__ sel_cnt, float *__restrict__ out, double *__restrict__ tau_out,
    float *__restrict__ weights_out, DecodeWs ws) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int kGroups = kDThreads / DIM;  // support entries processed in parallel
  __shared__ double dred[kDThreads / kWave];
  __shared__ int scan_scratch[kDThreads / kWave];
  __shared__ double qs[DIM];
  __shared__ int s_last;
  __shared__ size_t sup_off[kSupChunk];
  __shared__ float sup_w[kSupChunk];
  __shared__ float accs[kGroups][DIM];
  const int rows = D.B * D.Hq;
  int *prefix = reinterpret_cast<int *>(smem);
  double *xstage = reinterpret_cast<double *>(smem + (((rows + 1) * 4 + 15) & ~15));
  double *sortbuf = xstage + kStage;
  const int total = build_item_map(D, dp, seq_lens, sel_cnt, prefix, rows, scan_scratch);
  const int P = D.P;
  const size_t wrow = (size_t)D.max_pages * P;

  // rows without items: their results are defined here (no last block will come)
  for (int r = blockIdx.x; r < rows; r += gridDim.x) {
    bool bad;
    const int c = row_items(D, dp, seq_lens, sel_cnt, r, &bad);
    if (c != 0) continue;
    if (threadIdx.x == 0 && tau_out) tau_out[r] = NAN;
    for (int i = threadIdx.x; i < DIM; i += kDThreads) out[(size_t)r * DIM + i] = bad ? NAN : 0.0f;
    if (weights_out)
      for (size_t i = threadIdx.x; i < wrow; i += kDThreads) st_agent(&weights_out[(size_t)r * wrow + i], 0.0f);
  }

  const int parts = kDThreads / P;  // threads per token
  const int per = DIM / parts;      // coordinates per thread
  const int tok = threadIdx.x / parts, part = threadIdx.x % parts;
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int r = find_row(prefix, rows, item);
    const int i = item - prefix[r];
    const int b = r / D.Hq, h = r % D.Hq, g = h / D.G;
    const int L = seq_len_clamped(seq_lens, b, D);
    const int np = n_pages_of(L, P);
    bool row_bad;
    const int cnt = row_items(D, dp, seq_lens, sel_cnt, r, &row_bad);
    bool bad_item = false;
    int p = i, prev = i - 1;
    if (!dp.full) {
      p = sel_idx[(size_t)r * D.max_pages + i];
      prev = i > 0 ? sel_idx[(size_t)r * D.max_pages + i - 1] : -1;
      if (p < 0 || p >= np || prev >= p) bad_item = true;
    }
    int phys = -1;
    if (!bad_item) {
      phys = page_table[(size_t)b * D.max_pages + p];
      if (phys < 0 || phys >= D.num_phys) bad_item = true;
    }
    double *xrow = ws.xs + (size_t)r * wrow;
    __syncthreads();
    for (int t = threadIdx.x; t < DIM; t += kDThreads) qs[t] = (double)load_f<T>(q, (size_t)r * DIM + t);
    __syncthreads();
    if (bad_item) {
      if (threadIdx.x == 0) st_agent(&ws.badf[r], ws.epoch);  // benign race: every writer stores the epoch
      for (int j = threadIdx.x; j < P; j += kDThreads) st_agent(&xrow[(size_t)i * P + j], -INFINITY);
    } else {
      const int n = min(P, L - p * P);
      const T *kp = k_pool + (((size_t)phys * D.Hkv + g) * P + tok) * DIM + part * per;
      double acc = 0.0;
      if (tok < n) {
#pragma unroll 8
        for (int e = 0; e < per; ++e) acc = __builtin_fma((double)load_f<T>(kp, e), qs[part * per + e], acc);
      }
      for (int o = parts / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, kWave);
      if (part == 0) st_agent(&xrow[(size_t)i * P + tok], tok < n ? dp.a * (dp.c * acc) : -INFINITY);
      // weights_out: zero every slot of the pages this item covers, (prev, p]
      // (the last item also covers the pages after p); the support weights are
      // written later by the row's last block.
      if (weights_out) {
        const size_t lo_s = (size_t)(prev + 1) * P;
        const size_t hi_s = (i == cnt - 1) ? wrow : (size_t)(p + 1) * P;
        for (size_t s = lo_s + threadIdx.x; s < hi_s; s += kDThreads)
          st_agent(&weights_out[(size_t)r * wrow + s], 0.0f);
      }
    }
    if (!arrive_last_ep(&ws.ctr[r], ws.epoch, (unsigned)cnt, &s_last)) continue;

    // ================= last item of row r: threshold, normalizer, output
    const bool badrow = row_bad || ld_agent(&ws.badf[r]) == ws.epoch;
    if (badrow) {
      if (threadIdx.x == 0 && tau_out) tau_out[r] = NAN;
      for (int c2 = threadIdx.x; c2 < DIM; c2 += kDThreads) out[(size_t)r * DIM + c2] = NAN;
      continue;
    }
    const int nX = cnt * P;
    RowScores rs;
    rs.load(xrow, nX, xstage);
    double tau;
    if (dp.tau_method == 1 && dp.ibeta == 1 && nX <= kSortMax) tau = sparsemax_tau_sort(rs, sortbuf, dred);
    else tau = solve_tau(rs, dp, dred);
    double z = 0.0;
    rs.for_each([&](int, double x) {
      const double y = x - tau;
      if (y > 0.0) z += entw(y, dp);
    });
    z = block_sum(z, dred);
    if (threadIdx.x == 0 && tau_out) tau_out[r] = tau / dp.a;

    // support gather: compact (V row offset, weight, weight slot) in index
    // order, chunk by chunk.  The thread that takes an entry resolves its page
    // (one round of dependent loads, in parallel across entries); the groups of
    // DIM threads then add p_t * v_t with independent loads, in a fixed order.
    const int grp = threadIdx.x / DIM, c2 = threadIdx.x % DIM;
    float acc = 0.0f;
    int base_cnt = 0;
    auto flush = [&](int nsup) {
      __syncthreads();
      int e = grp;
      for (; e + 3 * kGroups < nsup; e += 4 * kGroups) {
        const float v0 = load_f<T>(v_pool, sup_off[e] + c2);
        const float v1 = load_f<T>(v_pool, sup_off[e + kGroups] + c2);
        const float v2 = load_f<T>(v_pool, sup_off[e + 2 * kGroups] + c2);
        const float v3 = load_f<T>(v_pool, sup_off[e + 3 * kGroups] + c2);
        acc += sup_w[e] * v0;
        acc += sup_w[e + kGroups] * v1;
        acc += sup_w[e + 2 * kGroups] * v2;
        acc += sup_w[e + 3 * kGroups] * v3;
      }
      for (; e < nsup; e += kGroups) acc += sup_w[e] * load_f<T>(v_pool, sup_off[e] + c2);
      __syncthreads();
    };
    auto take_entry = [&](int slot, int idx, float w) {
      const int it = idx / P, j = idx % P;
      const int pg = dp.full ? it : sel_idx[(size_t)r * D.max_pages + it];
      const int ph = page_table[(size_t)b * D.max_pages + pg];
      sup_off[slot] = (((size_t)ph * D.Hkv + g) * P + j) * DIM;
      sup_w[slot] = w;
      if (weights_out) st_agent(&weights_out[(size_t)r * wrow + (size_t)pg * P + j], w);
    };
    // in index order, one block-wide compaction step per 256 scores
#pragma unroll 1
    for (int i0 = 0; i0 < nX; i0 += kDThreads) {
      const int ii = i0 + threadIdx.x;
      const double y = (ii < nX ? rs.at(ii) : -INFINITY) - tau;
      const int take = y > 0.0 ? 1 : 0;
      int tot;
      const int pos = block_excl_scan(take, scan_scratch, &tot);
      if (base_cnt + tot > kSupChunk) { flush(base_cnt); base_cnt = 0; }
      if (take) take_entry(base_cnt + pos, ii, (float)(entw(y, dp) / z));
      base_cnt += tot;
    }
    flush(base_cnt);
    accs[grp][c2] = acc;
    __syncthreads();
    for (int cc = threadIdx.x; cc < DIM; cc += kDThreads) {
      float sacc = accs[0][cc];
      for (int gi = 1; gi < kGroups; ++gi) sacc += accs[gi][cc];
      out[(size_t)r * DIM + cc] = sacc;
    }
    __syncthreads();
  }
}

static DecodeWs carve_decode(const Dims &D, void *base, size_t *bytes) {
  Carve cv(base);
  const size_t rows = (size_t)D.B * D.Hq;
  DecodeWs w;
  w.xs = cv.take<double>(rows * D.max_pages * D.P);
  w.badf = cv.take<unsigned long long>(rows);
  w.ctr = cv.take<unsigned long long>(rows);
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
  const size_t smem = map_bytes + (size_t)kStage * sizeof(double) +
                      (dp.tau_method == 1 ? (size_t)kSortMax * sizeof(double) : 0);
  static bool attr_set = false;
  if (!attr_set) {
    // largest dynamic LDS any shape can ask for: item map of 8192 rows + stage + sort buffer
    hipFuncSetAttribute((const void *)entmax_decode_kernel<T, DIM>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)(((8193 * 4 + 15) & ~15) + (size_t)(kStage + kSortMax) * sizeof(double)));
    attr_set = true;
  }
  hipLaunchKernelGGL((entmax_decode_kernel<T, DIM>), dim3(kDGrid), dim3(kDThreads), smem, s, D, dp,
                     (const T *)q, (const T *)k_pool, (const T *)v_pool, page_table, seq_lens, sel_idx,
                     sel_cnt, out, tau, weights_out, w);
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
