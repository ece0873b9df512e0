// gauss.hip -- Gaussian-aware entmax page selection ([EntmaxKV s.2.B], policy 2).
//
// EntmaxKV s.2.B = section 2.B ("candidate selection policies") of "Resumen
// Tecnico: EntmaxKV - Decodificacion Consciente del Soporte para Atencion
// Entmax", gist.science/es/paper/2605.21649: estimate the global alpha-entmax
// threshold from the page-level Gaussian statistics by solving an approximate
// normalization equation, then keep the pages whose estimated maximum score
// exceeds that threshold adjusted by a safety margin Delta.
//
// Reading implemented here (the page gives no formulas):
//   F(t) = sum_p n_p sum_j w_j [a (mu_p + sqrt2 sigma_p x_j) - t]_+^beta,
//   a = alpha - 1, beta = 1/a, (x_j, w_j) 16-point Gauss-Hermite (w / sqrt(pi)),
//   tau_hat = root of F(tau_hat) = 1,
//   keep p  iff  min(mu_p + n_sigma sigma_p, box_p) >= tau_hat/a - Delta,
//   none kept -> keep the page of largest estimate (lowest index on ties).
//
// Root finding for beta in {1, 2} (alpha = 2, 1.5) without a sequential bisection
// over every point (16 per page):
//   K1  per (row, chunk): lower bracket lo with F(lo) >= 1, the larger of
//       max_p [a mu_p - (2.5/n_p)^a] (the page alone already gives F >= 1
//       there, since half of the rule's weight sits on nodes x_j >= 0) and
//       theta - W^-a for rule weight W of the chunk's points above theta
//       (eight thresholds theta below the top node); upper bracket hi =
//       max_p of the top node (F = 0 there).
//   K2  per (row, chunk): histogram of the points v > lo over NB equal bins of
//       [lo, hi] holding the moments M_r = sum c (v - e_b)^r, r <= beta, taken
//       about each bin's lower edge e_b.  The last block of a row merges the
//       chunks in order and runs a suffix scan of the moments (shifting them
//       edge to edge keeps every term non-negative, so there is no
//       cancellation): F at every edge follows exactly, which fixes the bin
//       [e_k, e_k+1) that holds the root.
//   K3  per (row, chunk): collect the points inside that bin, and classify each
//       page as kept / dropped / undecided for every threshold the bin allows.
//       The last block solves F = 1 inside the bin (suffix polynomial + the
//       collected points) by Newton steps from the left (F is convex and
//       decreasing), settles the undecided pages and writes the ascending list.
// Other alpha fall back to one block per row running a plain bisection.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace ekv {

constexpr int kGThreads = 256;
constexpr int kNB = 256;  // histogram bins
constexpr int kNThr = 3;  // thresholds of the certified lower bracket
constexpr int kZB = 128;  // buckets of the node lookup over z in [-5, 5)
constexpr double kZLo = -5.0, kZScale = kZB / 10.0;

// Suffix tables of the rule about each node and the node lookup (host-built):
// T_r[k] = sum_{j >= k} w_j (x_j - x_k)^r, so the rule weight of a page's
// points above theta is n T0[k] with k the first node above
// z = (theta - a mu) / (a sqrt2 sigma).
struct GaussTables {
  double t[17][4];        // T0[k], T1[k], T2[k], x_k (row 16: no node above, x = +inf)
  unsigned char kb[kZB];  // first node above the bucket's lower edge
};

// First node above z: bucket table plus one compare (a bucket holds at most one node).
__device__ __forceinline__ int node_above(double z, const double (*tab)[4], const unsigned char *kb) {
  const double zc = fmin(fmax((z - kZLo) * kZScale, 0.0), (double)(kZB - 1));
  const int k = kb[(int)zc];
  return k + ((z >= tab[k][3]) ? 1 : 0);
}

struct GaussParams {
  double a, beta, delta, nsig;
  int chunk;   // pages per chunk
  int nchunk;  // chunks per row (max over rows)
  int cap;     // in-bin capacity per row (points)
  int ibeta;   // 1, 2 or 0 (generic)
};

struct GaussWs {
  double *part;        // [rows][nchunk][2]   lo candidate, top node
  double *hist;        // [rows][nchunk][kNB][3]
  double *rowinfo;     // [rows][8]           k, lo, w, T0, T1, T2
  double *inbin;       // [rows][cap][2]      (v, c)
  int *inbin_cnt;      // [rows]
  int *list;           // [rows][max_pages]   page | undecided<<31, per chunk segments
  int *list_cnt;       // [rows][nchunk]
  double *amax;        // [rows][nchunk][2]   best estimate, its page
  unsigned int *ctr;   // [rows][2]
};

__device__ __forceinline__ bool page_valid(float bx, float m, float v) {
  return isfinite(bx) && isfinite(m) && isfinite(v);
}
__device__ __forceinline__ double powb(double x, int ibeta, double beta) {
  return ibeta == 2 ? x * x : (ibeta == 1 ? x : pow(x, beta));
}
// keep predicate at threshold thr (score units); sqrt-free form of mu + n sigma >= thr
__device__ __forceinline__ bool keep_at(double thr, double bx, double m, double s2, double nsig) {
  const double dd = thr - m;
  const bool g_ok = (dd <= 0.0) || (nsig * nsig * s2 >= dd * dd);
  return g_ok && bx >= thr;
}
__device__ __forceinline__ double bin_edge(double lo, double w, int b) { return lo + (double)b * w; }
// LDS slot of histogram bin b: neighbouring Gauss-Hermite nodes of one page
// land ~16-40 bins apart, so a plain layout sends the lanes of one atomic to
// the same LDS banks; XOR-ing the low bits with the high ones spreads them
// (a permutation of 0 .. kNB-1).
__device__ __forceinline__ int hslot(int b) { return b ^ ((b >> 4) & 15); }
// Bin of a point from the reciprocal width (the histogram and the in-bin
// collection compute iw = 1/w from the same w, so they agree on every point;
// a point may sit a rounding error below its bin's edge, which the moment
// algebra about the edge absorbs).
__device__ __forceinline__ int bin_of(double v, double lo, double iw) {
  int b = (int)((v - lo) * iw);
  return b < 0 ? 0 : (b >= kNB ? kNB - 1 : b);
}

// Quadrature point j of a page in (alpha-1)-scaled score units; every kernel
// evaluates it with this one expression, so they agree on each point's bits.
__device__ __forceinline__ double gh_point(double a, double m, double sig, double x) {
  return a * (m + 1.4142135623730951 * sig * x);
}

// The page statistics of pages pb .. pb+3 (clamped to p_end - 1; the caller
// masks pages past the end).
struct Pages4 {
  float bx[4], m[4], v2[4];
  __device__ __forceinline__ void load(const float *box, const float *mu, const float *var, size_t base, int pb,
                                       int p_end) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = min(pb + u, p_end - 1);
      bx[u] = box[base + p];
      m[u] = mu[base + p];
      v2[u] = var[base + p];
    }
  }
};

struct RowCtx {
  int row, b, L, np, nch;
  bool active;
};
__device__ __forceinline__ RowCtx row_ctx(const Dims &D, const GaussParams &gp, const int32_t *seq_lens,
                                          const uint8_t *seq_mask, int row) {
  RowCtx r;
  r.row = row;
  r.b = row / D.Hq;
  r.active = !(seq_mask && !seq_mask[r.b]);
  r.L = seq_len_clamped(seq_lens, r.b, D);
  r.np = n_pages_of(r.L, D.P);
  r.nch = (r.np + gp.chunk - 1) / gp.chunk;
  return r;
}

// ---------------------------------------------------------------- K1: brackets
__global__ __launch_bounds__(kGThreads) void gauss_bracket_kernel(Dims D, GaussParams gp, GaussConsts gc,
                                                                  GaussTables gt,
                                                                  const float *__restrict__ box,
                                                                  const float *__restrict__ mu,
                                                                  const float *__restrict__ var,
                                                                  const int32_t *__restrict__ seq_lens,
                                                                  const uint8_t *__restrict__ seq_mask,
                                                                  GaussWs ws) {
  __shared__ double red[kNThr * kGThreads / kWave];
  __shared__ double tab[17][4];
  __shared__ unsigned char kb[kZB];
  const int chunk = blockIdx.x;
  EKV_MARK(0, 0);
  const RowCtx rc = row_ctx(D, gp, seq_lens, seq_mask, blockIdx.y);
  if (!rc.active) return;
  if (chunk == 0 && threadIdx.x == 0) {
    ws.inbin_cnt[rc.row] = 0;
    ws.ctr[rc.row * 2 + 0] = 0;
    ws.ctr[rc.row * 2 + 1] = 0;
  }
  if (chunk >= rc.nch && chunk > 0) return;
  for (int i = threadIdx.x; i < 17 * 4; i += kGThreads) tab[i / 4][i % 4] = gt.t[i / 4][i % 4];
  for (int i = threadIdx.x; i < kZB; i += kGThreads) kb[i] = gt.kb[i];
  const size_t base = (size_t)rc.row * D.max_pages;
  const double pw_full = pow(2.5 / (double)D.P, gp.a);  // the lone-page bracket term of a full page
  const int p_begin = chunk * gp.chunk, p_end = min(rc.np, (chunk + 1) * gp.chunk);
  // pass 1 (each thread 4 consecutive pages): the single-page bound and the top node
  double lo_c = -INFINITY, top = -INFINITY;
  Pages4 pg;
#pragma unroll 1
  for (int p0 = p_begin; p0 < p_end; p0 += 4 * kGThreads) {
    const int pb = p0 + 4 * threadIdx.x;
    pg.load(box, mu, var, base, pb, p_end);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (pb + u >= p_end || !page_valid(pg.bx[u], pg.m[u], pg.v2[u])) continue;
      const int n = min(D.P, rc.L - (pb + u) * D.P);
      const double sig = sqrt(pg.v2[u] > 0.0f ? (double)pg.v2[u] : 0.0);
      lo_c = fmax(lo_c, gp.a * (double)pg.m[u] - (n == D.P ? pw_full : pow(2.5 / (double)n, gp.a)));
      top = fmax(top, gh_point(gp.a, (double)pg.m[u], sig, gc.x[15]));
    }
  }
  EKV_MARK(0, 1);
  {  // both block maxima with one pair of barriers
    lo_c = wave_max(lo_c);
    top = wave_max(top);
    constexpr int nw = kGThreads / kWave;
    const int w = threadIdx.x / kWave;
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) { red[w] = lo_c; red[nw + w] = top; }
    __syncthreads();
    lo_c = red[0];
    top = red[nw];
    for (int i = 1; i < nw; ++i) { lo_c = fmax(lo_c, red[i]); top = fmax(top, red[nw + i]); }
  }
  // pass 2, a tighter certified bound: with W the rule weight (n_p w_j) of the
  // chunk's points above theta = top - f (top - lo_c),
  // F(theta - W^-(alpha-1)) >= W (W^-(alpha-1))^(1/(alpha-1)) = 1, and F of the
  // row is at least F of the chunk.  Per page W is n T0[k] (one table lookup).
  double lo_b = lo_c;
  if (top > lo_c) {
    const double span = top - lo_c;
    constexpr double kFrac[kNThr] = {0.35, 0.42, 0.5};
    double W[kNThr];
#pragma unroll
    for (int j = 0; j < kNThr; ++j) W[j] = 0.0;
#pragma unroll 1
    for (int p0 = p_begin; p0 < p_end; p0 += 4 * kGThreads) {
      const int pb = p0 + 4 * threadIdx.x;
      if (p_end - p_begin > 4 * kGThreads) pg.load(box, mu, var, base, pb, p_end);  // else still loaded
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (pb + u >= p_end || !page_valid(pg.bx[u], pg.m[u], pg.v2[u])) continue;
        const double n = (double)min(D.P, rc.L - (pb + u) * D.P);
        const double am = gp.a * (double)pg.m[u];
        const double B = gp.a * 1.4142135623730951 * sqrt(pg.v2[u] > 0.0f ? (double)pg.v2[u] : 0.0);
        const double ib = B > 0.0 ? 1.0 / B : 0.0;
#pragma unroll
        for (int j = 0; j < kNThr; ++j) {
          const double th = top - span * kFrac[j];
          if (!(B > 0.0)) { W[j] += am > th ? n : 0.0; continue; }  // point mass at a mu
          const int k = node_above((th - am) * ib, tab, kb);
          W[j] += k < 16 ? n * tab[k][0] : 0.0;
        }
      }
    }
    block_sum_n<kNThr>(W, red);
#pragma unroll
    for (int j = 0; j < kNThr; ++j) {
      if (W[j] > 0.0) {
        const double th = top - span * kFrac[j];
        const double d = gp.ibeta == 2 ? 1.0 / sqrt(W[j]) : 1.0 / W[j];  // W^-(alpha-1), alpha in {1.5, 2}
        lo_b = fmax(lo_b, th - d - 1e-12 * fmax(1.0, fabs(top)));
      }
    }
  }
  EKV_MARK(0, 2);
  if (threadIdx.x == 0) {
    ws.part[((size_t)rc.row * gp.nchunk + chunk) * 2 + 0] = lo_b;
    ws.part[((size_t)rc.row * gp.nchunk + chunk) * 2 + 1] = top;
  }
}

__device__ __forceinline__ void row_bracket(const GaussParams &gp, const GaussWs &ws, const RowCtx &rc,
                                            double &lo, double &hi) {
  lo = -INFINITY;
  hi = -INFINITY;
  const int n = rc.nch > 0 ? rc.nch : 1;
  // every slot is loaded (independent of the row's length, so the loads issue
  // at once); slots past the row's chunks are ignored
#pragma unroll 8
  for (int c = 0; c < gp.nchunk; ++c) {
    const double l = ws.part[((size_t)rc.row * gp.nchunk + c) * 2 + 0];
    const double h = ws.part[((size_t)rc.row * gp.nchunk + c) * 2 + 1];
    if (c < n) { lo = fmax(lo, l); hi = fmax(hi, h); }
  }
  if (hi > -INFINITY && !(hi > lo)) hi = lo + fmax(1e-300, fabs(lo) * 1e-15);
}

// ------------------------------------------------------------- K2: histograms
__global__ __launch_bounds__(kGThreads) void gauss_hist_kernel(Dims D, GaussParams gp, GaussConsts gc,
                                                               const float *__restrict__ mu,
                                                               const float *__restrict__ var,
                                                               const float *__restrict__ box,
                                                               const int32_t *__restrict__ seq_lens,
                                                               const uint8_t *__restrict__ seq_mask,
                                                               GaussWs ws) {
  __shared__ double h0[kNB], h1[kNB], h2[kNB];
  __shared__ double s0[kNB], s1[kNB], s2[kNB];
  __shared__ int s_last, s_best;
  const int chunk = blockIdx.x;
  EKV_MARK(1, 0);
  const RowCtx rc = row_ctx(D, gp, seq_lens, seq_mask, blockIdx.y);
  if (!rc.active || chunk >= rc.nch) return;
  const size_t base = (size_t)rc.row * D.max_pages;
  const int p_end = min(rc.np, (chunk + 1) * gp.chunk);
  // the first pages' statistics are requested before the bracket, so the two
  // round trips overlap
  Pages4 pg0;
  pg0.load(box, mu, var, base, chunk * gp.chunk + 4 * threadIdx.x, p_end);
  double lo, hi;
  row_bracket(gp, ws, rc, lo, hi);
  if (!(hi > -INFINITY)) return;  // no valid page in the row
  EKV_MARK(1, 1);
  const double w = (hi - lo) / kNB, iw = 1.0 / w;
  const double sqrt2 = 1.4142135623730951;
  for (int i = threadIdx.x; i < kNB; i += kGThreads) h0[i] = h1[i] = h2[i] = 0.0;
  __syncthreads();
  // Each thread takes 4 consecutive pages and walks the nodes from the top
  // (a wave-uniform index, so the node constants sit in scalar registers);
  // the 4 pages advance together for instruction-level parallelism, and a
  // page drops out at its first node below lo (the nodes ascend in j).
#pragma unroll 1
  for (int p0 = chunk * gp.chunk; p0 < p_end; p0 += 4 * kGThreads) {
    const int pb = p0 + 4 * threadIdx.x;
    Pages4 pg = pg0;
    if (p0 != chunk * gp.chunk) pg.load(box, mu, var, base, pb, p_end);
    double mm[4], sg[4], nn[4];
    bool act[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      act[u] = pb + u < p_end && page_valid(pg.bx[u], pg.m[u], pg.v2[u]);
      mm[u] = (double)pg.m[u];
      sg[u] = sqrt(pg.v2[u] > 0.0f ? (double)pg.v2[u] : 0.0);
      nn[u] = (double)min(D.P, rc.L - (pb + u) * D.P);
    }
    // The four pages' chains are computed side by side without branches (a
    // page past its last node yields a value that is simply not added), and
    // the node loop is unrolled so its constants are loaded up front: a
    // scalar load inside the loop would make every pass wait for the LDS
    // atomics before it (both count in the same wait counter).
#pragma unroll
    for (int j = 15; j >= 0; --j) {
      const double xj = gc.x[j], wj = gc.w[j];
      double v[4], e[4], c[4];
      int hs[4];
      bool in[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v[u] = gh_point(gp.a, mm[u], sg[u], xj);
        in[u] = act[u] && v[u] > lo;
        act[u] = in[u];
        const int bn = bin_of(in[u] ? v[u] : lo, lo, iw);
        e[u] = v[u] - bin_edge(lo, w, bn);
        c[u] = nn[u] * wj;
        hs[u] = hslot(bn);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (in[u]) {
          atomicAdd(&h0[hs[u]], c[u]);
          atomicAdd(&h1[hs[u]], c[u] * e[u]);
          if (gp.ibeta == 2) atomicAdd(&h2[hs[u]], c[u] * e[u] * e[u]);
        }
      }
      if (!__any(in[0] || in[1] || in[2] || in[3])) break;
    }
  }
  __syncthreads();
  EKV_MARK(1, 2);
  double *hc = ws.hist + ((size_t)rc.row * gp.nchunk + chunk) * kNB * 3;
  for (int i = threadIdx.x; i < kNB; i += kGThreads) {
    st_agent(&hc[i * 3 + 0], h0[hslot(i)]);
    st_agent(&hc[i * 3 + 1], h1[hslot(i)]);
    st_agent(&hc[i * 3 + 2], h2[hslot(i)]);
  }
  if (!arrive_last(&ws.ctr[rc.row * 2 + 0], (unsigned)rc.nch, &s_last)) return;
  EKV_MARK(1, 3);

  // ---- last block of the row: merge chunks in order, suffix-scan the moments
  for (int i = threadIdx.x; i < kNB; i += kGThreads) {
    double a0 = 0.0, a1 = 0.0, a2 = 0.0;
    for (int c0 = 0; c0 < rc.nch; c0 += 16) {  // batches of 16 chunks: one round trip each
      double v[16][3];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int c = min(c0 + u, rc.nch - 1);
        const double *hh = ws.hist + ((size_t)rc.row * gp.nchunk + c) * kNB * 3 + i * 3;
        v[u][0] = ld_agent(&hh[0]);
        v[u][1] = ld_agent(&hh[1]);
        v[u][2] = ld_agent(&hh[2]);
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if (c0 + u < rc.nch) { a0 += v[u][0]; a1 += v[u][1]; a2 += v[u][2]; }
      }
    }
    s0[i] = a0;
    s1[i] = a1;
    s2[i] = a2;
  }
  __syncthreads();
  EKV_MARK(1, 4);
  // inclusive suffix scan, S_b = m_b (+) shift(S_{b+1}, e_{b+1} -> e_b) with
  // shift(M, e' -> e) = (M0, M1 + D M0, M2 + 2 D M1 + D^2 M0), D = e' - e
  // (associative): within each wave by shuffles, then each lane adds the
  // higher waves' suffix, combined top-down in a fixed order, shifted to its
  // edge.  One thread per bin (kGThreads == kNB).
  {
    static_assert(kGThreads == kNB, "one thread per bin");
    __shared__ double hd[kNB / kWave][3];  // each wave's own suffix at its first bin
    const int i = threadIdx.x, lane = i & (kWave - 1), wv = i / kWave;
    double n0 = s0[i], n1 = s1[i], n2 = s2[i];
#pragma unroll
    for (int dist = 1; dist < kWave; dist <<= 1) {
      const double t0 = __shfl_down(n0, dist, kWave), t1 = __shfl_down(n1, dist, kWave),
                   t2 = __shfl_down(n2, dist, kWave);
      if (lane + dist < kWave) {
        const double Dd = bin_edge(lo, w, i + dist) - bin_edge(lo, w, i);
        n0 += t0;
        n1 += t1 + Dd * t0;
        n2 += t2 + 2.0 * Dd * t1 + Dd * Dd * t0;
      }
    }
    if (lane == 0) { hd[wv][0] = n0; hd[wv][1] = n1; hd[wv][2] = n2; }
    __syncthreads();
    // suffix of the waves above this one, about the edge of the next wave's first bin
    double h0 = 0.0, h1 = 0.0, h2 = 0.0;
    for (int v = kNB / kWave - 1; v > wv; --v) {
      if (v < kNB / kWave - 1) {  // shift the running suffix from e_{64(v+1)} to e_{64 v}
        const double Dd = bin_edge(lo, w, (v + 1) * kWave) - bin_edge(lo, w, v * kWave);
        h2 = h2 + 2.0 * Dd * h1 + Dd * Dd * h0;
        h1 = h1 + Dd * h0;
      }
      h0 += hd[v][0];
      h1 += hd[v][1];
      h2 += hd[v][2];
    }
    if (wv < kNB / kWave - 1) {
      const double Dd = bin_edge(lo, w, (wv + 1) * kWave) - bin_edge(lo, w, i);
      n0 += h0;
      n1 += h1 + Dd * h0;
      n2 += h2 + 2.0 * Dd * h1 + Dd * Dd * h0;
    }
    __syncthreads();
    s0[i] = n0;
    s1[i] = n1;
    s2[i] = n2;
    __syncthreads();
  }
  // F(e_b) = s2[b] (beta 2) or s1[b] (beta 1); root bin = largest b with F >= 1
  if (threadIdx.x == 0) s_best = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < kNB; i += kGThreads) {
    const double F = gp.ibeta == 2 ? s2[i] : s1[i];
    if (F >= 1.0) atomicMax(&s_best, i);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int k = s_best;
    double *ri = ws.rowinfo + (size_t)rc.row * 8;
    ri[0] = (double)k;
    ri[1] = lo;
    ri[2] = w;
    // moments of the bins above k, about e_{k+1}
    ri[3] = k + 1 < kNB ? s0[k + 1] : 0.0;
    ri[4] = k + 1 < kNB ? s1[k + 1] : 0.0;
    ri[5] = k + 1 < kNB ? s2[k + 1] : 0.0;
  }
  EKV_MARK(1, 5);
}

// F = 1 inside the root bin [ek, ek1] for rows with at most kWave * kBinReg
// in-bin points, on one wave (no block barriers): Newton from the left, and
// each pass also solves its piece exactly.  With A the in-bin points above t
// and every point of the bins above active (moments T about ek1),
// F(t + u) = f - fp u + q u^2 (beta 2, q = sum_A c + T0) or f - fp u (beta 1)
// until u reaches the nearest active in-bin point; the smaller root of
// F(t + u) = 1, when it stays below that point and inside the bin, is F's root.
constexpr int kBinReg = 8;
__device__ double bin_root_wave(const double (&v)[kBinReg], const double (&c)[kBinReg], double ek, double ek1,
                                double T0, double T1, double T2, int ibeta) {
  double t = ek;
#pragma unroll 1
  for (int it = 0; it < 200; ++it) {
    double f = 0.0, fp = 0.0, qa = 0.0, nmn = -INFINITY;
#pragma unroll
    for (int u = 0; u < kBinReg; ++u) {
      const double x = v[u] - t;
      if (x > 0.0) {
        if (ibeta == 2) { f += c[u] * x * x; fp += 2.0 * c[u] * x; }
        else { f += c[u] * x; fp += c[u]; }
        qa += c[u];
        nmn = fmax(nmn, -x);
      }
    }
    f = wave_sum(f);
    fp = wave_sum(fp);
    qa = wave_sum(qa);
    nmn = wave_max(nmn);
    const double Dd = ek1 - t;  // >= 0
    if (ibeta == 2) { f += T2 + 2.0 * Dd * T1 + Dd * Dd * T0; fp += 2.0 * T1 + 2.0 * Dd * T0; }
    else { f += T1 + Dd * T0; fp += T0; }
    if (!(fp > 0.0)) break;
    if (f > 1.0) {
      const double q = qa + T0;
      const double u = ibeta == 2 ? (f - 1.0) / (0.5 * fp + sqrt(fmax(0.25 * fp * fp - q * (f - 1.0), 0.0)))
                                  : (f - 1.0) / fp;
      if (u <= -nmn && t + u <= ek1) return t + u;
    }
    double tn = t + (f - 1.0) / fp;
    if (tn > ek1) tn = ek1;
    if (!(tn > t)) break;  // converged from the left (or rounding stalls)
    t = tn;
  }
  return t;
}

// --------------------------------------- K3: collect, classify, solve, compact
__global__ __launch_bounds__(kGThreads) void gauss_select_kernel(
    Dims D, GaussParams gp, GaussConsts gc, const float *__restrict__ box, const float *__restrict__ mu,
    const float *__restrict__ var, const int32_t *__restrict__ seq_lens,
    const uint8_t *__restrict__ seq_mask, int32_t *__restrict__ sel_idx, int32_t *__restrict__ sel_cnt,
    double *__restrict__ tau_hat, GaussWs ws) {
  __shared__ int scan_scratch[kGThreads / kWave];
  __shared__ double dred[3 * kGThreads / kWave];  // up to three block sums at once
  __shared__ double s_best_est;
  __shared__ int s_best_p, s_last;
  const int chunk = blockIdx.x;
  EKV_MARK(2, 0);
  const RowCtx rc = row_ctx(D, gp, seq_lens, seq_mask, blockIdx.y);
  if (!rc.active) return;
  const size_t base = (size_t)rc.row * D.max_pages;
  const int p_begin = chunk * gp.chunk, p_end = min(rc.np, (chunk + 1) * gp.chunk);
  // independent reads first, so their round trips overlap: this chunk's first
  // page statistics, the root bin and width, the bracket
  Pages4 pg0;
  if (chunk < rc.nch) pg0.load(box, mu, var, base, p_begin + 4 * threadIdx.x, p_end);
  const double *ri = ws.rowinfo + (size_t)rc.row * 8;
  const double ri_k = ri[0], ri_w = ri[2];
  double lo, hi;
  row_bracket(gp, ws, rc, lo, hi);
  if (!(hi > -INFINITY)) {  // no pages (or none valid): empty selection
    if (chunk == 0 && threadIdx.x == 0) {
      sel_cnt[rc.row] = 0;
      if (tau_hat) tau_hat[rc.row] = NAN;
    }
    return;
  }
  if (chunk >= rc.nch) return;
  EKV_MARK(2, 1);
  const int k = (int)ri_k;
  const double w = ri_w, iw = 1.0 / w;
  const double ek = bin_edge(lo, w, k), ek1 = bin_edge(lo, w, k + 1);
  const double thr_lo = ek / gp.a - gp.delta, thr_hi = ek1 / gp.a - gp.delta;
  const double sqrt2 = 1.4142135623730951;

  // ---- collect in-bin points and classify this chunk's pages (ascending order)
  int listed = 0;
  double best = -INFINITY;
  int bestp = 0x7FFFFFFF;
  // Each thread takes 4 consecutive pages (one block scan per 1024 pages
  // keeps the list ascending); the nodes are walked from the top with a
  // wave-uniform index and a page drops out below bin k.
#pragma unroll 1
  for (int p0 = p_begin; p0 < p_end; p0 += 4 * kGThreads) {
    const int pb = p0 + 4 * threadIdx.x;
    Pages4 pg = pg0;
    if (p0 != p_begin) pg.load(box, mu, var, base, pb, p_end);
    double mm[4], sg[4], s2d[4], nn[4];
    bool valid[4], act[4];
    int code[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = pb + u;
      valid[u] = p < p_end && page_valid(pg.bx[u], pg.m[u], pg.v2[u]);
      act[u] = valid[u];
      mm[u] = (double)pg.m[u];
      s2d[u] = pg.v2[u] > 0.0f ? (double)pg.v2[u] : 0.0;
      sg[u] = sqrt(s2d[u]);
      nn[u] = (double)min(D.P, rc.L - p * D.P);
      code[u] = -1;
      if (valid[u]) {
        if (keep_at(thr_hi, pg.bx[u], pg.m[u], s2d[u], gp.nsig)) code[u] = p;
        else if (keep_at(thr_lo, pg.bx[u], pg.m[u], s2d[u], gp.nsig)) code[u] = p | (int)0x80000000;
        const double e1 = mm[u] + gp.nsig * sg[u];
        const double est = e1 < (double)pg.bx[u] ? e1 : (double)pg.bx[u];
        if (est > best || (est == best && p < bestp)) { best = est; bestp = p; }
      }
    }
    // In-bin points take slots from one counter per row.  When many pages
    // share their statistics (a flat score distribution) thousands of points
    // fall into the root bin, so the slots are claimed per wave: one atomic
    // for the wave's points at a node, lane offsets from the ballot masks.
#pragma unroll 1
    for (int j = 15; j >= 0; --j) {
      const double xj = gc.x[j], wj = gc.w[j];
      bool any = false;
      bool in[4];
      double vin[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        in[u] = false;
        vin[u] = 0.0;
        if (!act[u]) continue;
        const double v = gh_point(gp.a, mm[u], sg[u], xj);
        const int bn = v > lo ? bin_of(v, lo, iw) : -1;
        if (bn < k) { act[u] = false; continue; }
        any = true;
        in[u] = bn == k;
        vin[u] = v;
      }
      int off[4], wave_tot = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const unsigned long long m = __ballot(in[u]);
        off[u] = wave_tot + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
        wave_tot += __popcll(m);
      }
      if (wave_tot > 0) {  // wave-uniform
        int slot0 = 0;
        if ((threadIdx.x & (kWave - 1)) == 0) slot0 = atomicAdd(&ws.inbin_cnt[rc.row], wave_tot);
        slot0 = __shfl(slot0, 0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int slot = slot0 + off[u];
          if (in[u] && slot < gp.cap) {
            st_agent(&ws.inbin[((size_t)rc.row * gp.cap + slot) * 2 + 0], vin[u]);
            st_agent(&ws.inbin[((size_t)rc.row * gp.cap + slot) * 2 + 1], nn[u] * wj);
          }
        }
      }
      if (!__any(any)) break;
    }
    int mine = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) mine += code[u] != -1 ? 1 : 0;
    int tot;
    int at = listed + block_excl_scan(mine, scan_scratch, &tot);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (code[u] != -1) st_agent(&ws.list[base + p_begin + at++], code[u]);
    listed += tot;
  }
  EKV_MARK(2, 2);
  // chunk argmax of the estimate (lowest page on ties)
  {
    double bm = block_max(best, dred);
    int cand = (best == bm) ? bestp : 0x7FFFFFFF;
    __syncthreads();
    if (threadIdx.x == 0) s_best_p = 0x7FFFFFFF;
    __syncthreads();
    if (cand != 0x7FFFFFFF) atomicMin(&s_best_p, cand);
    __syncthreads();
    if (threadIdx.x == 0) {
      st_agent(&ws.amax[((size_t)rc.row * gp.nchunk + chunk) * 2 + 0], bm);
      st_agent(&ws.amax[((size_t)rc.row * gp.nchunk + chunk) * 2 + 1], (double)s_best_p);
      st_agent(&ws.list_cnt[(size_t)rc.row * gp.nchunk + chunk], listed);
    }
  }
  if (!arrive_last(&ws.ctr[rc.row * 2 + 1], (unsigned)rc.nch, &s_last)) return;
  EKV_MARK(2, 3);

  // ---- last block of the row: solve F(t) = 1 inside [ek, ek1].  Up to
  // kWave * kBinReg in-bin points: one wave holds them in registers and solves
  // alone; more: the block holds kInReg per thread, any excess re-read per pass.
  const int nin = min(ld_agent(&ws.inbin_cnt[rc.row]), gp.cap);
  const double T0 = ri[3], T1 = ri[4], T2 = ri[5];
  const double *inb = ws.inbin + (size_t)rc.row * gp.cap * 2;
  EKV_MARK(2, 4);
  __shared__ double s_tbin;
  double t = ek;
  if (nin <= kWave * kBinReg) {
    if (threadIdx.x < kWave) {
      double wv[kBinReg], wc[kBinReg];
#pragma unroll
      for (int u = 0; u < kBinReg; ++u) {  // lane-strided copies of the points staged above
        const int i = u * kWave + (int)threadIdx.x;
        const int ic = min(i, max(nin - 1, 0));
        const double v = ld_agent(&inb[ic * 2 + 0]), c = ld_agent(&inb[ic * 2 + 1]);
        wv[u] = i < nin ? v : -INFINITY;
        wc[u] = i < nin ? c : 0.0;
      }
      const double tw = bin_root_wave(wv, wc, ek, ek1, T0, T1, T2, gp.ibeta);
      if (threadIdx.x == 0) s_tbin = tw;
    }
    __syncthreads();
    t = s_tbin;
  } else {
  // more points: the block holds kInReg per thread, any excess is re-read per pass
  constexpr int kInReg = 8;
  double rv[kInReg], rcw[kInReg];
#pragma unroll
  for (int u = 0; u < kInReg; ++u) {
    const int i = u * kGThreads + threadIdx.x;
    const int ic = min(i, max(nin - 1, 0));
    const double v = ld_agent(&inb[ic * 2 + 0]), c = ld_agent(&inb[ic * 2 + 1]);
    rv[u] = i < nin ? v : -INFINITY;
    rcw[u] = i < nin ? c : 0.0;
  }
  // Newton from the left, and each pass also solves its piece exactly: with
  // A the in-bin points above t and every point of the bins above active,
  // F(t + u) = f - fp u + q u^2 (beta 2, q = sum_A c + T0) or f - fp u
  // (beta 1) until u reaches the nearest active in-bin point, so the smaller
  // root u of F(t + u) = 1, when it stays below that point and inside the
  // bin, is F's root and ends the search.
  for (int it = 0; it < 200; ++it) {
    double sm[3] = {0.0, 0.0, 0.0};  // f, fp, sum_A c over the in-bin points
    double nmn = -INFINITY;          // -(distance to the nearest active in-bin point)
    auto acc_pt = [&](double v, double c) {
      const double x = v - t;
      if (x > 0.0) {
        if (gp.ibeta == 2) { sm[0] += c * x * x; sm[1] += 2.0 * c * x; }
        else { sm[0] += c * x; sm[1] += c; }
        sm[2] += c;
        nmn = fmax(nmn, -x);
      }
    };
#pragma unroll
    for (int u = 0; u < kInReg; ++u) acc_pt(rv[u], rcw[u]);
    for (int i = kInReg * kGThreads + threadIdx.x; i < nin; i += kGThreads)
      acc_pt(ld_agent(&inb[i * 2 + 0]), ld_agent(&inb[i * 2 + 1]));
    block_sum_n<3>(sm, dred);
    nmn = block_max(nmn, dred);
    double f = sm[0], fp = sm[1];
    const double Dd = ek1 - t;  // >= 0
    if (gp.ibeta == 2) { f += T2 + 2.0 * Dd * T1 + Dd * Dd * T0; fp += 2.0 * T1 + 2.0 * Dd * T0; }
    else { f += T1 + Dd * T0; fp += T0; }
    if (!(fp > 0.0)) break;
    if (f > 1.0) {
      const double q = sm[2] + T0;
      const double u = gp.ibeta == 2 ? (f - 1.0) / (0.5 * fp + sqrt(fmax(0.25 * fp * fp - q * (f - 1.0), 0.0)))
                                     : (f - 1.0) / fp;
      if (u <= -nmn && t + u <= ek1) {
        t = t + u;
        break;
      }
    }
    double tn = t + (f - 1.0) / fp;
    if (tn > ek1) tn = ek1;
    if (!(tn > t)) break;  // converged from the left (or rounding stalls)
    t = tn;
  }
  }
  const double tau = t;
  if (threadIdx.x == 0) {
    if (tau_hat) tau_hat[rc.row] = tau / gp.a;
    ws.inbin_cnt[rc.row] = 0;
  }
  const double thr = tau / gp.a - gp.delta;


  EKV_MARK(2, 5);  // ---- settle undecided pages and write the ascending list.  Chunk counts
  // and argmax partials are fetched in one batch; list entries are then read
  // in parallel across chunks (prefix offsets in LDS).
  __shared__ int s_off[1024 + 1];
  __shared__ double s_ae[1024];
  __shared__ int s_ap[1024];
  for (int c = threadIdx.x; c < rc.nch; c += kGThreads) {
    s_off[c + 1] = ld_agent(&ws.list_cnt[(size_t)rc.row * gp.nchunk + c]);
    s_ae[c] = ld_agent(&ws.amax[((size_t)rc.row * gp.nchunk + c) * 2 + 0]);
    s_ap[c] = (int)ld_agent(&ws.amax[((size_t)rc.row * gp.nchunk + c) * 2 + 1]);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    s_off[0] = 0;
    for (int c = 0; c < rc.nch; ++c) s_off[c + 1] += s_off[c];
  }
  __syncthreads();
  const int n_listed = s_off[rc.nch];
  EKV_MARK(2, 6);
  int total = 0;
  for (int e0 = 0; e0 < n_listed; e0 += kGThreads) {
    const int e = e0 + threadIdx.x;
    int take = 0, p = 0;
    if (e < n_listed) {
      int lo_c = 0, hi_c = rc.nch - 1;  // chunk holding entry e
      while (lo_c < hi_c) {
        const int mid = (lo_c + hi_c + 1) >> 1;
        if (s_off[mid] <= e) lo_c = mid; else hi_c = mid - 1;
      }
      const int code = ld_agent(&ws.list[base + (size_t)lo_c * gp.chunk + (e - s_off[lo_c])]);
      p = code & 0x7FFFFFFF;
      if (code >= 0) take = 1;
      else {
        const float m = mu[base + p], v2 = var[base + p];
        take = keep_at(thr, (double)box[base + p], (double)m, v2 > 0.0f ? (double)v2 : 0.0, gp.nsig) ? 1 : 0;
      }
    }
    int tot;
    const int pos = block_excl_scan(take, scan_scratch, &tot);
    if (take) sel_idx[base + total + pos] = p;
    total += tot;
  }
  if (threadIdx.x == 0) {
    if (total == 0) {
      double be = -INFINITY;
      int bp = 0x7FFFFFFF;
      for (int c = 0; c < rc.nch; ++c) {
        if (s_ap[c] == 0x7FFFFFFF) continue;
        if (bp == 0x7FFFFFFF || s_ae[c] > be) { be = s_ae[c]; bp = s_ap[c]; }
      }
      sel_idx[base] = bp;
      total = 1;
    }
    sel_cnt[rc.row] = total;
  }
}

// ---------------------------------------------- generic alpha: one block / row
constexpr int kGenThreads = 1024;
__global__ __launch_bounds__(kGenThreads) void gauss_generic_kernel(
    Dims D, GaussParams gp, GaussConsts gc, const float *__restrict__ box, const float *__restrict__ mu,
    const float *__restrict__ var, const int32_t *__restrict__ seq_lens,
    const uint8_t *__restrict__ seq_mask, int32_t *__restrict__ sel_idx, int32_t *__restrict__ sel_cnt,
    double *__restrict__ tau_hat) {
  __shared__ double dred[kGenThreads / kWave];
  __shared__ int scan_scratch[kGenThreads / kWave];
  __shared__ int s_best_p;
  const RowCtx rc = row_ctx(D, gp, seq_lens, seq_mask, blockIdx.x);
  if (!rc.active) return;
  const size_t base = (size_t)rc.row * D.max_pages;
  const double sqrt2 = 1.4142135623730951;
  double mumax = -INFINITY, top = -INFINITY;
  for (int p = threadIdx.x; p < rc.np; p += kGenThreads) {
    const float bx = box[base + p], m = mu[base + p], v2 = var[base + p];
    if (!page_valid(bx, m, v2)) continue;
    mumax = fmax(mumax, (double)m);
    top = fmax(top, gp.a * ((double)m + sqrt2 * sqrt(v2 > 0.0f ? (double)v2 : 0.0) * gc.x[15]));
  }
  mumax = block_max(mumax, dred);
  top = block_max(top, dred);
  if (!(top > -INFINITY)) {
    if (threadIdx.x == 0) {
      sel_cnt[rc.row] = 0;
      if (tau_hat) tau_hat[rc.row] = NAN;
    }
    return;
  }
  auto F = [&](double t) {
    double f = 0.0;
    for (int p = threadIdx.x; p < rc.np; p += kGenThreads) {
      const float bx = box[base + p], m = mu[base + p], v2 = var[base + p];
      if (!page_valid(bx, m, v2)) continue;
      const double n = (double)min(D.P, rc.L - p * D.P);
      const double sig = sqrt(v2 > 0.0f ? (double)v2 : 0.0);
      double inner = 0.0;
      for (int j = 0; j < 16; ++j) {
        const double x = gp.a * ((double)m + sqrt2 * sig * gc.x[j]) - t;
        if (x > 0.0) inner += gc.w[j] * powb(x, gp.ibeta, gp.beta);
      }
      f += n * inner;
    }
    return block_sum(f, dred);
  };
  double gap = 1.0, lo = gp.a * mumax - gap;
  while (F(lo) < 1.0) { gap *= 2.0; lo = gp.a * mumax - gap; }
  double hi = top;
  for (int it = 0; it < 2100; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (mid == lo || mid == hi) break;
    if (F(mid) >= 1.0) lo = mid; else hi = mid;
  }
  if (threadIdx.x == 0 && tau_hat) tau_hat[rc.row] = lo / gp.a;
  const double thr = lo / gp.a - gp.delta;
  int total = 0;
  double best = -INFINITY;
  int bestp = 0x7FFFFFFF;
  for (int p0 = 0; p0 < rc.np; p0 += kGenThreads) {
    const int p = p0 + threadIdx.x;
    int take = 0;
    if (p < rc.np) {
      const float bx = box[base + p], m = mu[base + p], v2 = var[base + p];
      if (page_valid(bx, m, v2)) {
        const double s2d = v2 > 0.0f ? (double)v2 : 0.0;
        take = keep_at(thr, bx, m, s2d, gp.nsig) ? 1 : 0;
        const double e1 = (double)m + gp.nsig * sqrt(s2d);
        const double est = e1 < (double)bx ? e1 : (double)bx;
        if (est > best) { best = est; bestp = p; }
      }
    }
    int tot;
    const int pos = block_excl_scan(take, scan_scratch, &tot);
    if (take) sel_idx[base + total + pos] = p;
    total += tot;
  }
  const double bm = block_max(best, dred);
  if (threadIdx.x == 0) s_best_p = 0x7FFFFFFF;
  __syncthreads();
  if (best == bm && bestp != 0x7FFFFFFF) atomicMin(&s_best_p, bestp);
  __syncthreads();
  if (threadIdx.x == 0) {
    if (total == 0) {
      sel_idx[base] = s_best_p;
      total = 1;
    }
    sel_cnt[rc.row] = total;
  }
}

// ----------------------------------------------------------------------- host
static GaussParams make_params(const Dims &D, double alpha, double delta, double n_sigma) {
  GaussParams gp;
  gp.a = alpha - 1.0;
  gp.beta = 1.0 / gp.a;
  gp.delta = delta;
  gp.nsig = n_sigma;
  gp.ibeta = alpha == 1.5 ? 2 : (alpha == 2.0 ? 1 : 0);
  const int rows = D.B * D.Hq;
  // enough chunks to give the GPU ~512 blocks, at least 256 pages per chunk
  int want = (512 + rows - 1) / rows;
  int chunk = (D.max_pages + want - 1) / want;
  chunk = ((chunk + 255) / 256) * 256;
  if (chunk < 256) chunk = 256;
  gp.chunk = chunk;
  gp.nchunk = (D.max_pages + chunk - 1) / chunk;
  if (gp.nchunk > 1024) {  // the selection kernel stages per-chunk data for up to 1024 chunks
    gp.chunk = ((D.max_pages + 1023) / 1024 + 255) / 256 * 256;
    gp.nchunk = (D.max_pages + gp.chunk - 1) / gp.chunk;
  }
  gp.cap = 16 * D.max_pages;
  return gp;
}

static GaussWs carve_gauss(const Dims &D, const GaussParams &gp, void *base, size_t *bytes) {
  Carve cv(base);
  const size_t rows = (size_t)D.B * D.Hq;
  GaussWs w;
  w.part = cv.take<double>(rows * gp.nchunk * 2);
  w.hist = cv.take<double>(rows * gp.nchunk * kNB * 3);
  w.rowinfo = cv.take<double>(rows * 8);
  w.inbin = cv.take<double>(rows * (size_t)gp.cap * 2);
  w.inbin_cnt = cv.take<int>(rows);
  w.list = cv.take<int>(rows * (size_t)D.max_pages);
  w.list_cnt = cv.take<int>(rows * gp.nchunk);
  w.amax = cv.take<double>(rows * gp.nchunk * 2);
  w.ctr = cv.take<unsigned int>(rows * 2);
  if (bytes) *bytes = cv.bytes();
  return w;
}

static GaussTables build_tables(const GaussConsts &gc) {
  GaussTables gt;
  for (int k = 0; k <= 16; ++k) {
    double t0 = 0.0, t1 = 0.0, t2 = 0.0;
    for (int j = k; j < 16; ++j) {
      const double dx = gc.x[j] - gc.x[k];
      t0 += gc.w[j];
      t1 += gc.w[j] * dx;
      t2 += gc.w[j] * dx * dx;
    }
    gt.t[k][0] = t0;
    gt.t[k][1] = t1;
    gt.t[k][2] = t2;
    gt.t[k][3] = k < 16 ? gc.x[k] : INFINITY;
  }
  for (int b = 0; b < kZB; ++b) {
    const double edge = kZLo + b / kZScale;
    int k = 0;
    while (k < 16 && gc.x[k] <= edge) ++k;
    gt.kb[b] = (unsigned char)k;
  }
  return gt;
}

size_t gauss_ws_bytes(const Dims &D) {
  GaussParams gp = make_params(D, 1.5, 0.0, 3.0);
  size_t bytes = 0;
  carve_gauss(D, gp, nullptr, &bytes);
  return bytes;
}

hipError_t launch_gauss(const Dims &D, const float *box, const float *mu, const float *var,
                        const int32_t *seq_lens, double alpha, double delta, double n_sigma,
                        const uint8_t *seq_mask, int32_t *sel_idx, int32_t *sel_cnt,
                        double *tau_hat, void *ws, hipStream_t s) {
  const GaussParams gp = make_params(D, alpha, delta, n_sigma);
  const GaussConsts &gc = gauss_consts();
  const int rows = D.B * D.Hq;
  if (gp.ibeta == 0) {
    hipLaunchKernelGGL(gauss_generic_kernel, dim3(rows), dim3(kGenThreads), 0, s, D, gp, gc, box, mu,
                       var, seq_lens, seq_mask, sel_idx, sel_cnt, tau_hat);
    return hipGetLastError();
  }
  GaussWs w = carve_gauss(D, gp, ws, nullptr);
  dim3 grid(gp.nchunk, rows);
  static const GaussTables gt = build_tables(gc);
  hipLaunchKernelGGL(gauss_bracket_kernel, grid, dim3(kGThreads), 0, s, D, gp, gc, gt, box, mu, var,
                     seq_lens, seq_mask, w);
  hipLaunchKernelGGL(gauss_hist_kernel, grid, dim3(kGThreads), 0, s, D, gp, gc, mu, var, box, seq_lens,
                     seq_mask, w);
  hipLaunchKernelGGL(gauss_select_kernel, grid, dim3(kGThreads), 0, s, D, gp, gc, box, mu, var,
                     seq_lens, seq_mask, sel_idx, sel_cnt, tau_hat, w);
  return hipGetLastError();
}

EKV_TRACE_DUMP(ekv_trace_dump_gauss)
}  // namespace ekv
