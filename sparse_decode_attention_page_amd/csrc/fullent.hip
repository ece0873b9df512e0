// fullent.hip -- full-cache alpha-entmax decode: the second baseline of the
// EntmaxKV summary's efficiency results ("Resumen Tecnico: EntmaxKV ...",
// gist.science/es/paper/2605.21649, section 4): alpha-entmax attention over
// every cached token.
//
// Two launches:
//  A  stream K once (split-K ranges of pages, all G query heads of a KV group
//     from the same bytes).  Exact fp64 scores; X = (alpha-1) s is stored as
//     float32 for filtering, and every range records the exact maximum of X.
//  B  per (row, chunk of tokens): tau >= max X - 1 (the top token alone gives
//     F >= 1 there), so only tokens with X above that bound can be in the
//     support.  The candidates (a margin covers the float32 rounding) are
//     listed per chunk; the last chunk-block of a row recomputes their scores
//     exactly, solves tau, and gathers V rows of the support tokens only.
// V is therefore read only where p_t > 0.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace ekv {

constexpr int kFThreads = 256;
constexpr int kFChunk = 16384;  // tokens per filtering block
constexpr int kFCache = 16;     // candidates staged per thread in the last block

struct FullWs {
  float *xf;                // [rows][max_pages*P]   X as float32 (-inf past the end)
  double *rmax;             // [rows][S]             exact max X of each range
  int *cand;                // [rows][max_pages*P]   candidate tokens, per-chunk segments
  int *cand_cnt;            // [rows][nchunk]
  double *cx;               // [rows][max_pages*P]   exact X of the candidates (last block scratch)
  int *ctok;                // [rows][max_pages*P]   their tokens, compacted (last block scratch)
  unsigned long long *ctr;  // [rows]
  unsigned long long epoch;
  int S, pps, nchunk;
};

struct FullParams {
  double a, beta, c;
  int ibeta;
};

__device__ __forceinline__ double fentw(double x, const FullParams &fp) {
  return fp.ibeta == 2 ? x * x : (fp.ibeta == 1 ? x : pow(x, fp.beta));
}
__device__ __forceinline__ double fentw_d(double x, const FullParams &fp) {
  return fp.ibeta == 2 ? 2.0 * x : (fp.ibeta == 1 ? 1.0 : fp.beta * pow(x, fp.beta - 1.0));
}

// ------------------------------------------------------------------ A: scores
template <typename T, int DIM, int P, int G>
__global__ __launch_bounds__(kFThreads) void full_scores_kernel(Dims D, FullParams fp, const T *__restrict__ q,
                                                                const T *__restrict__ k_pool,
                                                                const int32_t *__restrict__ page_table,
                                                                const int32_t *__restrict__ seq_lens, FullWs ws) {
  constexpr int kParts = kFThreads / P;
  constexpr int kPer = DIM / kParts;
  constexpr int kWords = kPer * (int)sizeof(T) / 4;
  __shared__ double smax[kFThreads / kWave][G];
  __shared__ int s_badrange;
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, slot = tid / kParts, part = tid % kParts;
  const int L = seq_len_clamped(seq_lens, b, D);
  const int np = n_pages_of(L, P);
  const int p_begin = s * ws.pps, p_end = min(np, (s + 1) * ws.pps);
  const size_t wrow = (size_t)D.max_pages * P;

  double qv[G][kPer];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < kPer; ++e)
      qv[h][e] = (double)load_f<T>(q, ((size_t)b * D.Hq + g * G + h) * DIM + part * kPer + e);
  double mx[G];
#pragma unroll
  for (int h = 0; h < G; ++h) mx[h] = -INFINITY;

  auto phys_of = [&](int p) {
    const int ph = page_table[(size_t)b * D.max_pages + p];
    return (ph < 0 || ph >= D.num_phys) ? -1 : ph;
  };
  if (tid == 0) s_badrange = 0;
  __syncthreads();
  uint32_t kw[kWords];
  int p = p_begin;
  int ph = p < p_end ? phys_of(p) : -1;
  if (ph >= 0) {
    const uint32_t *kp = reinterpret_cast<const uint32_t *>(k_pool + (((size_t)ph * D.Hkv + g) * P + slot) * DIM + part * kPer);
#pragma unroll
    for (int w = 0; w < kWords; ++w) kw[w] = kp[w];
  }
  for (; p < p_end; ++p) {
    uint32_t nk[kWords];
    const int pn = p + 1;
    const int phn = pn < p_end ? phys_of(pn) : -1;
    if (phn >= 0) {
      const uint32_t *kp = reinterpret_cast<const uint32_t *>(k_pool + (((size_t)phn * D.Hkv + g) * P + slot) * DIM + part * kPer);
#pragma unroll
      for (int w = 0; w < kWords; ++w) nk[w] = kp[w];
    }
    double kd[kPer];
#pragma unroll
    for (int w = 0; w < kWords; ++w) {
      if constexpr (sizeof(T) == 2) {
        kd[2 * w] = bf16lo(kw[w]);
        kd[2 * w + 1] = bf16hi(kw[w]);
      } else {
        kd[w] = __uint_as_float(kw[w]);
      }
    }
    double sc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      double a = 0.0;
#pragma unroll
      for (int e = 0; e < kPer; ++e) a = __builtin_fma(qv[h][e], kd[e], a);  // exact products
      sc[h] = a;
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int o = kParts / 2; o > 0; o >>= 1) sc[h] += __shfl_xor(sc[h], o, kWave);
    const int t = p * P + slot;
    const bool live = ph >= 0 && t < L;
    if (ph < 0) s_badrange = 1;  // benign race: every writer stores 1
    if (part == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const double x = fp.a * (fp.c * sc[h]);
        const float xs = live ? (float)x : (ph < 0 ? NAN : -INFINITY);
        ws.xf[((size_t)b * D.Hq + g * G + h) * wrow + t] = xs;
        if (live) mx[h] = fmax(mx[h], x);
      }
    }
    ph = phn;
#pragma unroll
    for (int w = 0; w < kWords; ++w) kw[w] = nk[w];
  }
  // exact range maxima (NaN poisons a range that met a bad page id)
#pragma unroll
  for (int h = 0; h < G; ++h) mx[h] = wave_max(mx[h]);
  const int wave = tid / kWave, lane = tid % kWave;
  if (lane == 0)
#pragma unroll
    for (int h = 0; h < G; ++h) smax[wave][h] = mx[h];
  __syncthreads();
  if (tid < G) {
    double m = smax[0][tid];
    for (int w = 1; w < kFThreads / kWave; ++w) m = fmax(m, smax[w][tid]);
    ws.rmax[((size_t)b * D.Hq + g * G + tid) * ws.S + s] = s_badrange ? NAN : m;
  }
}

// --------------------------------------------- B: filter, solve, gather support
template <typename T, int DIM>
__global__ __launch_bounds__(kFThreads) void full_select_kernel(Dims D, FullParams fp, const T *__restrict__ q,
                                                                const T *__restrict__ k_pool,
                                                                const T *__restrict__ v_pool,
                                                                const int32_t *__restrict__ page_table,
                                                                const int32_t *__restrict__ seq_lens,
                                                                float *__restrict__ out, double *__restrict__ tau_out,
                                                                float *__restrict__ weights_out, FullWs ws) {
  __shared__ double dred[kFThreads / kWave];
  __shared__ int scan_scratch[kFThreads / kWave];
  __shared__ int s_last, s_bad;
  __shared__ double s_M;
  __shared__ int s_off[1024 + 1];
  __shared__ double qs[DIM];
  constexpr int kGroups = kFThreads / DIM;
  __shared__ float accs[kGroups][DIM];
  __shared__ int sup_t[1024];
  __shared__ float sup_w[1024];
  const int chunk = blockIdx.x, row = blockIdx.y;
  const int b = row / D.Hq, h = row % D.Hq, g = h / D.G;
  const int L = seq_len_clamped(seq_lens, b, D);
  const int P = D.P;
  const size_t wrow = (size_t)D.max_pages * P;
  const int nch = (L + kFChunk - 1) / kFChunk;
  if (L == 0) {
    if (chunk == 0) {
      for (int i = threadIdx.x; i < DIM; i += kFThreads) out[(size_t)row * DIM + i] = 0.0f;
      if (threadIdx.x == 0 && tau_out) tau_out[row] = NAN;
      if (weights_out)
        for (size_t i = threadIdx.x; i < wrow; i += kFThreads) weights_out[(size_t)row * wrow + i] = 0.0f;
    }
    return;
  }
  if (chunk >= nch) return;
  // row maximum from the range maxima (exact), NaN = bad page id somewhere
  const int S_used = (n_pages_of(L, P) + ws.pps - 1) / ws.pps;
  double m = -INFINITY;
  bool bad = false;
  for (int s = threadIdx.x; s < S_used; s += kFThreads) {
    const double v = ws.rmax[(size_t)row * ws.S + s];
    if (v != v) bad = true;
    m = fmax(m, v);
  }
  m = block_max(m, dred);
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  if (bad) s_bad = 1;
  __syncthreads();
  const bool row_bad = s_bad != 0;
  // candidates: X > M - 1 can be in the support; the float32 copy may be low by
  // 2^-24 |X|, so keep everything within that margin
  const double bound = m - 1.0 - 1e-6 * fmax(1.0, fabs(m));
  const int t0 = chunk * kFChunk, t1 = min(L, t0 + kFChunk);
  const float *xr = ws.xf + (size_t)row * wrow;
  int *cseg = ws.cand + (size_t)row * wrow + t0;
  int listed = 0;
  for (int base = t0; base < t1; base += kFThreads) {
    const int t = base + threadIdx.x;
    const int take = (t < t1 && (double)xr[t] > bound) ? 1 : 0;
    int tot;
    const int pos = block_excl_scan(take, scan_scratch, &tot);
    if (take) st_agent(&cseg[listed + pos], t);
    listed += tot;
  }
  if (threadIdx.x == 0) st_agent(&ws.cand_cnt[(size_t)row * ws.nchunk + chunk], listed);
  if (weights_out)
    for (int t = t0 + threadIdx.x; t < t0 + kFChunk && (size_t)t < wrow; t += kFThreads)
      st_agent(&weights_out[(size_t)row * wrow + t], 0.0f);
  if (weights_out && chunk == nch - 1)
    for (size_t t = (size_t)nch * kFChunk + threadIdx.x; t < wrow; t += kFThreads)
      st_agent(&weights_out[(size_t)row * wrow + t], 0.0f);
  if (!arrive_last_ep(&ws.ctr[row], ws.epoch, (unsigned)nch, &s_last)) return;

  // ================= last block of the row
  if (row_bad) {
    for (int i = threadIdx.x; i < DIM; i += kFThreads) out[(size_t)row * DIM + i] = NAN;
    if (threadIdx.x == 0 && tau_out) tau_out[row] = NAN;
    return;
  }
  for (int c = threadIdx.x; c < nch; c += kFThreads) s_off[c + 1] = ld_agent(&ws.cand_cnt[(size_t)row * ws.nchunk + c]);
  for (int i = threadIdx.x; i < DIM; i += kFThreads) qs[i] = (double)load_f<T>(q, (size_t)row * DIM + i);
  __syncthreads();
  if (threadIdx.x == 0) {
    s_off[0] = 0;
    for (int c = 0; c < nch; ++c) s_off[c + 1] += s_off[c];
  }
  __syncthreads();
  const int ncand = s_off[nch];
  double *cx = ws.cx + (size_t)row * wrow;
  // exact scores of the candidates, in chunk (= token) order
  for (int e = threadIdx.x; e < ncand; e += kFThreads) {
    int lo_c = 0, hi_c = nch - 1;
    while (lo_c < hi_c) {
      const int mid = (lo_c + hi_c + 1) >> 1;
      if (s_off[mid] <= e) lo_c = mid; else hi_c = mid - 1;
    }
    const int t = ld_agent(&ws.cand[(size_t)row * wrow + (size_t)lo_c * kFChunk + (e - s_off[lo_c])]);
    const int ph = page_table[(size_t)b * D.max_pages + t / P];
    const T *kr = k_pool + (((size_t)ph * D.Hkv + g) * P + t % P) * DIM;
    double acc = 0.0;
    for (int i = 0; i < DIM; ++i) acc += (double)load_f<T>(kr, i) * qs[i];
    cx[e] = fp.a * (fp.c * acc);
    ws.ctok[(size_t)row * wrow + e] = t;
  }
  __syncthreads();
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // tau: safeguarded Newton from the left over the candidates
  auto for_each = [&](auto &&fn) {
    for (int e = threadIdx.x; e < ncand; e += kFThreads) fn(e, cx[e]);
  };
  double mx = -INFINITY, cnt = 0.0;
  for_each([&](int, double x) { mx = fmax(mx, x); cnt += 1.0; });
  mx = block_max(mx, dred);
  double lo = mx - 1.0;
  double hi = mx - pow((double)L, -fp.a);
  bool bisect_next = false;
  for (int it = 0; it < 400 && hi > lo; ++it) {
    double cand;
    if (bisect_next) {
      cand = 0.5 * (lo + hi);
    } else {
      double f = 0.0, fd = 0.0;
      for_each([&](int, double x) {
        const double y = x - lo;
        if (y > 0.0) { f += fentw(y, fp); fd += fentw_d(y, fp); }
      });
      f = block_sum(f, dred);
      fd = block_sum(fd, dred);
      cand = fd > 0.0 ? lo + (f - 1.0) / fd : 0.5 * (lo + hi);
      if (!(cand > lo) || !(cand < hi)) {
        if (!(cand > lo) && f >= 1.0) break;
        cand = 0.5 * (lo + hi);
      }
    }
    if (cand == lo || cand == hi) break;
    double f = 0.0;
    for_each([&](int, double x) {
      const double y = x - cand;
      if (y > 0.0) f += fentw(y, fp);
    });
    f = block_sum(f, dred);
    if (f >= 1.0) { lo = cand; bisect_next = false; }
    else { hi = cand; bisect_next = true; }
  }
  const double tau = lo;
  double z = 0.0;
  for_each([&](int, double x) {
    const double y = x - tau;
    if (y > 0.0) z += fentw(y, fp);
  });
  z = block_sum(z, dred);
  if (threadIdx.x == 0 && tau_out) tau_out[row] = tau / fp.a;
  // support gather in token order
  const int grp = threadIdx.x / DIM, c2 = threadIdx.x % DIM;
  float acc = 0.0f;
  int nsup = 0;
  for (int e0 = 0; e0 < ncand; e0 += kFThreads) {
    const int e = e0 + threadIdx.x;
    double y = -1.0;
    if (e < ncand) y = cx[e] - tau;
    const int take = y > 0.0 ? 1 : 0;
    int tot;
    const int pos = block_excl_scan(take, scan_scratch, &tot);
    if (nsup + tot > 1024) {
      __syncthreads();
      for (int k = grp; k < nsup; k += kGroups) {
        const int t = sup_t[k];
        const int ph = page_table[(size_t)b * D.max_pages + t / P];
        acc += sup_w[k] * load_f<T>(v_pool + (((size_t)ph * D.Hkv + g) * P + t % P) * DIM, c2);
      }
      __syncthreads();
      nsup = 0;
    }
    if (take) {
      const int t = ws.ctok[(size_t)row * wrow + e];
      sup_t[nsup + pos] = t;
      const float w = (float)(fentw(y, fp) / z);
      sup_w[nsup + pos] = w;
      if (weights_out) st_agent(&weights_out[(size_t)row * wrow + t], w);
    }
    nsup += tot;
  }
  __syncthreads();
  for (int k = grp; k < nsup; k += kGroups) {
    const int t = sup_t[k];
    const int ph = page_table[(size_t)b * D.max_pages + t / P];
    acc += sup_w[k] * load_f<T>(v_pool + (((size_t)ph * D.Hkv + g) * P + t % P) * DIM, c2);
  }
  accs[grp][c2] = acc;
  __syncthreads();
  for (int cc = threadIdx.x; cc < DIM; cc += kFThreads) {
    float sacc = accs[0][cc];
    for (int gi = 1; gi < kGroups; ++gi) sacc += accs[gi][cc];
    out[(size_t)row * DIM + cc] = sacc;
  }
}

static FullWs carve_full(const Dims &D, void *base, size_t *bytes) {
  FullWs w;
  const int bg = D.B * D.Hkv;
  int S = (1024 + bg - 1) / bg;
  const int maxS = (D.max_pages + 7) / 8;
  if (S > maxS) S = maxS;
  if (S < 1) S = 1;
  w.S = S;
  w.pps = (D.max_pages + S - 1) / S;
  const size_t wrow = (size_t)D.max_pages * D.P;
  w.nchunk = (int)((wrow + kFChunk - 1) / kFChunk);
  const size_t rows = (size_t)D.B * D.Hq;
  Carve cv(base);
  w.xf = cv.take<float>(rows * wrow);
  w.rmax = cv.take<double>(rows * S);
  w.cand = cv.take<int>(rows * wrow);
  w.cand_cnt = cv.take<int>(rows * w.nchunk);
  w.cx = cv.take<double>(rows * wrow);
  w.ctok = cv.take<int>(rows * wrow);
  w.ctr = cv.take<unsigned long long>(rows);
  w.epoch = 0;
  if (bytes) *bytes = cv.bytes();
  return w;
}

size_t full_ws_bytes(const Dims &D) {
  size_t b = 0;
  carve_full(D, nullptr, &b);
  return b;
}

template <typename T, int DIM, int P, int G>
static hipError_t launch_full_t(const Dims &D, const FullParams &fp, const void *q, const void *k, const void *v,
                                const int32_t *pt, const int32_t *sl, float *out, double *tau, float *wout,
                                FullWs w, hipStream_t s) {
  hipLaunchKernelGGL((full_scores_kernel<T, DIM, P, G>), dim3(w.S, D.Hkv, D.B), dim3(kFThreads), 0, s, D, fp,
                     (const T *)q, (const T *)k, pt, sl, w);
  hipLaunchKernelGGL((full_select_kernel<T, DIM>), dim3(w.nchunk, D.B * D.Hq), dim3(kFThreads), 0, s, D, fp,
                     (const T *)q, (const T *)k, (const T *)v, pt, sl, out, tau, wout, w);
  return hipGetLastError();
}

template <typename T, int DIM, int P>
static hipError_t launch_full_g(const Dims &D, const FullParams &fp, const void *q, const void *k, const void *v,
                                const int32_t *pt, const int32_t *sl, float *out, double *tau, float *wout,
                                FullWs w, hipStream_t s) {
  switch (D.G) {
    case 1: return launch_full_t<T, DIM, P, 1>(D, fp, q, k, v, pt, sl, out, tau, wout, w, s);
    case 2: return launch_full_t<T, DIM, P, 2>(D, fp, q, k, v, pt, sl, out, tau, wout, w, s);
    case 4: return launch_full_t<T, DIM, P, 4>(D, fp, q, k, v, pt, sl, out, tau, wout, w, s);
    case 8: return launch_full_t<T, DIM, P, 8>(D, fp, q, k, v, pt, sl, out, tau, wout, w, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, int DIM>
static hipError_t launch_full_p(const Dims &D, const FullParams &fp, const void *q, const void *k, const void *v,
                                const int32_t *pt, const int32_t *sl, float *out, double *tau, float *wout,
                                FullWs w, hipStream_t s) {
  switch (D.P) {
    case 16: return launch_full_g<T, DIM, 16>(D, fp, q, k, v, pt, sl, out, tau, wout, w, s);
    case 32: return launch_full_g<T, DIM, 32>(D, fp, q, k, v, pt, sl, out, tau, wout, w, s);
    case 64: return launch_full_g<T, DIM, 64>(D, fp, q, k, v, pt, sl, out, tau, wout, w, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_entmax_full(const Dims &D, int dtype, const void *q, const void *k_pool, const void *v_pool,
                              const int32_t *page_table, const int32_t *seq_lens, double alpha, float *out,
                              double *tau, float *weights_out, void *ws, hipStream_t s) {
  FullWs w = carve_full(D, ws, nullptr);
  w.epoch = next_epoch();
  FullParams fp;
  fp.a = alpha - 1.0;
  fp.beta = 1.0 / fp.a;
  fp.c = D.scale;
  fp.ibeta = alpha == 1.5 ? 2 : (alpha == 2.0 ? 1 : 0);
  if (dtype == ENTMAXKV_BF16) {
    if (D.d == 64) return launch_full_p<uint16_t, 64>(D, fp, q, k_pool, v_pool, page_table, seq_lens, out, tau, weights_out, w, s);
    return launch_full_p<uint16_t, 128>(D, fp, q, k_pool, v_pool, page_table, seq_lens, out, tau, weights_out, w, s);
  }
  if (D.d == 64) return launch_full_p<float, 64>(D, fp, q, k_pool, v_pool, page_table, seq_lens, out, tau, weights_out, w, s);
  return launch_full_p<float, 128>(D, fp, q, k_pool, v_pool, page_table, seq_lens, out, tau, weights_out, w, s);
}

}  // namespace ekv
