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
// F is a sum over the row's quadrature points y_pj = a (mu_p + sqrt2 sigma_p
// x_j) with weights c_pj = n_p w_j; it is convex and decreasing in t.
//
// Root finding for beta in {1, 2} (alpha = 2, 1.5), in three launches over
// (row, chunk of pages), every sum in a fixed order so that tau_hat and the set
// are the same bits on every run:
//   K1  bracket: lo = max_p [a mu_p - (2.5/n_p)^a] (the page alone gives
//       F >= 1.25 there: half of the rule's weight sits on nodes x_j >= 0) and
//       hi = the largest point (F = 0 there); per chunk, merged by max.
//   K2  counts: the points above lo fall into kNB equal bins of [lo, hi]; each
//       block counts n_p per (node, bin) in LDS and adds its counts to the row's
//       with integer atomics (integer sums do not depend on the order).  The
//       row's last block turns the counts into the exact bin weights W_b =
//       sum_j w_j N_bj and bounds F at every bin edge e_b from below and above
//       (a point of bin b' lies in [e_b', e_b'+1)); the root lies in the window
//       [e_lo, e_hi) between the last edge certified F >= 1 and the first
//       certified F < 1, usually two or three bins.
//   K3  solve: every block adds the moments of its points above e_hi about e_hi
//       (per page of a thread, pages combined in order, then a fixed-order block sum), lists its points
//       inside the window in page order, and classifies its pages as kept /
//       dropped / undecided for any threshold in the window.  The row's last
//       block adds the chunks' moments in chunk order, solves F = 1 on the
//       window (Newton from the left, each pass also solving the current piece
//       of F exactly), settles the undecided pages and writes the ascending set.
// Other alpha fall back to one block per row running a plain bisection.
#include <math.h>

#include <cmath>

#include "common.hpp"
#include "launch.hpp"

namespace ekv {

constexpr int kGThreads = 256;
constexpr int kGroup = 4 * kGThreads;  // pages per group: 4 consecutive pages per thread
#ifndef EKV_GAUSS_NB
#define EKV_GAUSS_NB 512
#endif
constexpr int kNB = EKV_GAUSS_NB;      // count bins over [lo, hi] (even, <= 2 kGThreads)
constexpr int kNodes = 16;
constexpr int kMaxChunks = 1024;       // chunk partials staged in LDS by the last blocks
constexpr int kWinReg = 8;             // window points per lane in the one-wave solve
constexpr int kBlkReg = 8;             // window points per thread in registers in the block solve
constexpr double kCertEps = 1e-9;      // relative safety of the certified edge bounds
#ifndef EKV_GAUSS_BLOCKS
#define EKV_GAUSS_BLOCKS 512           // blocks the (row, chunk) grid aims at
#endif

struct GaussParams {
  double a, beta, delta, nsig;
  double lone_full;  // (2.5/P)^a
  int chunk;         // pages per chunk (a multiple of kGroup or kGroup itself)
  int nchunk;        // chunk slots per row (max over rows)
  int ibeta;         // 1, 2 or 0 (generic)
  int rows;
  int vec;           // box/mu/var 16-byte aligned and max_pages % 4 == 0
  int sum_tiles;     // 0: the bracket launch's chunk partials; else the scorer's summary, entries per row
};

struct GaussWs {
  unsigned *cnt;     // [rows][kNodes][kNB] sum of n_p over the points of node j in bin b
  unsigned *ctr;     // [rows][2]          arrival counters of K2 and K3 (zeroed by K1)
  double *part;      // [rows][nchunk][2]  chunk max of the lone-page bound, chunk's largest point
  const double *summ;  // [rows][sum_tiles][2] the scorer's bracket terms (when sum_tiles > 0)
  int *win;          // [rows][2]          window bins k_lo, k_hi
  double *mom;       // [rows][nchunk][3]  moments above e_hi about e_hi
  int *wcnt;         // [rows][nchunk]     window points per chunk
  int *wpts;         // [rows][max_pages * kNodes] window points (page * 16 + node), chunk segments
  int *list;         // [rows][max_pages]  kept / undecided pages (undecided: bit 31), chunk segments
  int *lcnt;         // [rows][nchunk]
  double *amax;      // [rows][nchunk][2]  chunk's largest estimate and its page
};

__device__ __forceinline__ bool page_valid(float bx, float m, float v) {
  return isfinite(bx) && isfinite(m) && isfinite(v);
}
__device__ __forceinline__ double powb(double x, int ibeta, double beta) {
  return ibeta == 2 ? x * x : (ibeta == 1 ? x : pow(x, beta));
}
// keep predicate at threshold thr (score units); sqrt-free form of mu + n sigma >= thr.
// Monotone in thr: true at thr implies true at every smaller thr.
__device__ __forceinline__ bool keep_at(double thr, double bx, double m, double s2, double nsig) {
  const double dd = thr - m;
  const bool g_ok = (dd <= 0.0) || (nsig * nsig * s2 >= dd * dd);
  return g_ok && bx >= thr;
}
// Quadrature point of a page in (alpha-1)-scaled score units; every kernel
// evaluates it with this one expression, so they agree on each point's bits.
__device__ __forceinline__ double gh_point(double a, double m, double sig, double x) {
  return a * (m + 1.4142135623730951 * sig * x);
}
__device__ __forceinline__ double sigma_of(float v2) { return sqrt(v2 > 0.0f ? (double)v2 : 0.0); }
// (2.5/n)^a for alpha in {1.5, 2}
__device__ __forceinline__ double lone_gap(int n, const GaussParams &gp) {
  if (gp.ibeta == 2) return sqrt(2.5 / (double)n);
  return 2.5 / (double)n;
}

// Blocks of a row share an XCD: workgroup L runs on XCD L % 8, so row r's
// chunks take the launch slots L with L % 8 == r % 8 (their reads of the
// row's statistics hit the same L2 in all three launches).
struct RowChunk {
  int row, chunk;
  bool ok;
};
__device__ __forceinline__ RowChunk map_block(int L, const GaussParams &gp) {
  const int xcd = L & 7, slot = L >> 3;
  const int rl = slot / gp.nchunk;
  RowChunk rc;
  rc.chunk = slot - rl * gp.nchunk;
  rc.row = rl * 8 + xcd;
  rc.ok = rc.row < gp.rows;
  return rc;
}
static int grid_of(const GaussParams &gp) { return ((gp.rows + 7) / 8) * 8 * gp.nchunk; }

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

// The statistics of pages p .. p+3 of a row (entries past max_pages read the
// row's last entry; the caller masks pages past the end).
struct Pages4 {
  float bx[4], m[4], v2[4];
  __device__ __forceinline__ void load(const float *box, const float *mu, const float *var, size_t base, int p,
                                       const Dims &D, const GaussParams &gp) {
    if (gp.vec && p + 4 <= D.max_pages) {
      const float4 b4 = *reinterpret_cast<const float4 *>(box + base + p);
      const float4 m4 = *reinterpret_cast<const float4 *>(mu + base + p);
      const float4 v4 = *reinterpret_cast<const float4 *>(var + base + p);
      bx[0] = b4.x; bx[1] = b4.y; bx[2] = b4.z; bx[3] = b4.w;
      m[0] = m4.x; m[1] = m4.y; m[2] = m4.z; m[3] = m4.w;
      v2[0] = v4.x; v2[1] = v4.y; v2[2] = v4.z; v2[3] = v4.w;
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = min(p + u, D.max_pages - 1);
        bx[u] = box[base + q];
        m[u] = mu[base + q];
        v2[u] = var[base + q];
      }
    }
  }
};

// Row bracket from the chunk partials (or from the scorer's summary: the
// largest mean over full pages and the largest top point, per 64-page tile;
// the last page, when partial, adds its own lone-page bound): every thread
// loads its share (all in flight at once), then a block max (max does not
// depend on the order).  Called by every thread of the block; red holds
// 2 kGThreads / kWave doubles.
__device__ __forceinline__ void row_bracket(const Dims &D, const GaussParams &gp, const GaussWs &ws,
                                            const RowCtx &rc, const float *box, const float *mu,
                                            const float *var, double &lo, double &hi, double *red) {
  double l = -INFINITY, h = -INFINITY;
  if (gp.sum_tiles) {
    const int nt = (rc.np + kSummaryTile - 1) / kSummaryTile;
    for (int c = threadIdx.x; c < nt; c += kGThreads) {
      const double2 v = *reinterpret_cast<const double2 *>(ws.summ + ((size_t)rc.row * gp.sum_tiles + c) * 2);
      l = fmax(l, v.x);
      h = fmax(h, v.y);
    }
  } else {
    for (int c = threadIdx.x; c < rc.nch; c += kGThreads) {
      const double2 v = *reinterpret_cast<const double2 *>(ws.part + ((size_t)rc.row * gp.nchunk + c) * 2);
      l = fmax(l, v.x);
      h = fmax(h, v.y);
    }
  }
  l = wave_max(l);
  h = wave_max(h);
  constexpr int nw = kGThreads / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    red[threadIdx.x / kWave] = l;
    red[nw + threadIdx.x / kWave] = h;
  }
  __syncthreads();
  lo = red[0];
  hi = red[nw];
#pragma unroll
  for (int i = 1; i < nw; ++i) {
    lo = fmax(lo, red[i]);
    hi = fmax(hi, red[nw + i]);
  }
  if (gp.sum_tiles) {
    lo = gp.a * lo - gp.lone_full;
    hi = gp.a * hi;
    const int nlast = rc.L - (rc.np - 1) * D.P;
    if (rc.np > 0 && nlast < D.P) {
      const size_t i = (size_t)rc.row * D.max_pages + rc.np - 1;
      const float bx = box[i], m = mu[i], v2 = var[i];
      if (page_valid(bx, m, v2)) lo = fmax(lo, gp.a * (double)m - lone_gap(nlast, gp));
    }
  }
}
// Bin edges: e_b = lo + b w for b < kNB, e_kNB = hi.
__device__ __forceinline__ double edge(double lo, double hi, double w, int b) {
  return b >= kNB ? hi : lo + (double)b * w;
}
// ---------------------------------------------------------------- K1: bracket
__global__ __launch_bounds__(kGThreads) void gauss_bracket_kernel(Dims D, GaussParams gp, GaussConsts gc,
                                                                  const float *__restrict__ box,
                                                                  const float *__restrict__ mu,
                                                                  const float *__restrict__ var,
                                                                  const int32_t *__restrict__ seq_lens,
                                                                  const uint8_t *__restrict__ seq_mask,
                                                                  GaussWs ws) {
  __shared__ double red[2 * kGThreads / kWave];
  const RowChunk bc = map_block(blockIdx.x, gp);
  if (!bc.ok) return;
  EKV_MARK(0, 0);
  const RowCtx rc = row_ctx(D, gp, seq_lens, seq_mask, bc.row);
  if (!rc.active) return;
  const int tid = threadIdx.x, chunk = bc.chunk;
  // this row's counts and arrival counters start at zero (every chunk slot
  // clears a share, also slots past the row's chunks)
  {
    uint4 *c4 = reinterpret_cast<uint4 *>(ws.cnt + (size_t)rc.row * kNodes * kNB);
    for (int i = chunk * kGThreads + tid; i < kNodes * kNB / 4; i += gp.nchunk * kGThreads)
      c4[i] = make_uint4(0u, 0u, 0u, 0u);
    if (chunk == 0 && tid < 2) ws.ctr[rc.row * 2 + tid] = 0u;
  }
  if (chunk >= rc.nch) return;
  const size_t base = (size_t)rc.row * D.max_pages;
  const int p_end = min(rc.np, (chunk + 1) * gp.chunk);
  double lo_c = -INFINITY, top = -INFINITY;
#pragma unroll 1
  for (int p0 = chunk * gp.chunk + 4 * tid; p0 < p_end; p0 += kGroup) {
    Pages4 pg;
    pg.load(box, mu, var, base, p0, D, gp);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = p0 + u;
      if (p >= p_end || !page_valid(pg.bx[u], pg.m[u], pg.v2[u])) continue;
      const int n = min(D.P, rc.L - p * D.P);
      const double m = (double)pg.m[u];
      lo_c = fmax(lo_c, gp.a * m - (n == D.P ? gp.lone_full : lone_gap(n, gp)));
      top = fmax(top, gh_point(gp.a, m, sigma_of(pg.v2[u]), gc.x[15]));
    }
  }
  EKV_MARK(0, 1);
  lo_c = wave_max(lo_c);
  top = wave_max(top);
  constexpr int nw = kGThreads / kWave;
  if ((tid & (kWave - 1)) == 0) {
    red[tid / kWave] = lo_c;
    red[nw + tid / kWave] = top;
  }
  __syncthreads();
  if (tid == 0) {
    for (int i = 1; i < nw; ++i) {
      lo_c = fmax(lo_c, red[i]);
      top = fmax(top, red[nw + i]);
    }
    ws.part[((size_t)rc.row * gp.nchunk + chunk) * 2 + 0] = lo_c;
    ws.part[((size_t)rc.row * gp.nchunk + chunk) * 2 + 1] = top;
  }
}

// Inclusive suffix sums Z_r(b) = sum_{b' >= b} (b' - b)^r W_b' (r = 0, 1, 2) of
// the bins, two consecutive bins per thread (threads past kNB / 2 hold empty
// pairs).  Combining
// a range with the suffix that starts d bins after its start shifts that
// suffix: Z0 + Z0', Z1 + Z1' + d Z0', Z2 + Z2' + 2 d Z1' + d^2 Z0' -- every
// term non-negative, so there is no cancellation.
struct Z3 {
  double z0, z1, z2;
};
__device__ __forceinline__ Z3 z_shift_add(const Z3 &a, const Z3 &s, double d) {
  return Z3{a.z0 + s.z0, a.z1 + (s.z1 + d * s.z0), a.z2 + (s.z2 + 2.0 * d * s.z1 + d * d * s.z0)};
}

// ----------------------------------------------------------------- K2: counts
__global__ __launch_bounds__(kGThreads) void gauss_count_kernel(Dims D, GaussParams gp, GaussConsts gc,
                                                                const float *__restrict__ box,
                                                                const float *__restrict__ mu,
                                                                const float *__restrict__ var,
                                                                const int32_t *__restrict__ seq_lens,
                                                                const uint8_t *__restrict__ seq_mask,
                                                                GaussWs ws) {
  static_assert(kNB % 4 == 0 && kNB <= 2 * kGThreads, "two bins per thread in the window search");
  __shared__ __align__(16) unsigned hc[kNodes * kNB];  // [node][bin]
  __shared__ Z3 s_wave[kGThreads / kWave];
  __shared__ double s_red[2 * kGThreads / kWave];
  __shared__ double s_w1[kGThreads];
  __shared__ double s_gx[kNodes];
  __shared__ int s_last, s_klo, s_khi;
  const RowChunk bc = map_block(blockIdx.x, gp);
  if (!bc.ok) return;
  EKV_MARK(1, 0);
  const RowCtx rc = row_ctx(D, gp, seq_lens, seq_mask, bc.row);
  const int tid = threadIdx.x, chunk = bc.chunk;
  if (!rc.active || chunk >= rc.nch) return;
  const size_t base = (size_t)rc.row * D.max_pages;
  const int p_begin = chunk * gp.chunk, p_end = min(rc.np, p_begin + gp.chunk);
  // independent loads first: this chunk's first pages and the row's bracket
  Pages4 pg0;
  pg0.load(box, mu, var, base, p_begin + 4 * tid, D, gp);
  if (tid < kNodes) s_gx[tid] = gc.x[tid];  // read in the node loop below (ordered by row_bracket's barrier)
  double lo, hi;
  row_bracket(D, gp, ws, rc, box, mu, var, lo, hi, s_red);
  if (!(hi > -INFINITY)) return;  // no valid page: K3 writes the empty result
  const double w = (hi - lo) / kNB, iw = 1.0 / w;
  {
    uint4 *h4 = reinterpret_cast<uint4 *>(hc);
    for (int i = tid; i < kNodes * kNB / 4; i += kGThreads) h4[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  EKV_MARK(1, 1);
  // Each thread takes 4 consecutive pages and walks the nodes from the top (a
  // wave-uniform node index, so the node constants are scalars); a page drops
  // out at its first point at or below lo (the points ascend with the node).
#pragma unroll 1
  for (int p0 = p_begin + 4 * tid; p0 - 4 * tid < p_end; p0 += kGroup) {
    Pages4 pg = pg0;
    if (p0 != p_begin + 4 * tid) pg.load(box, mu, var, base, p0, D, gp);
    double mm[4], sg[4];
    unsigned nn[4];
    bool act[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = p0 + u;
      act[u] = p < p_end && page_valid(pg.bx[u], pg.m[u], pg.v2[u]);
      mm[u] = (double)pg.m[u];
      sg[u] = sigma_of(pg.v2[u]);
      nn[u] = (unsigned)max(0, min(D.P, rc.L - p * D.P));
    }
    // (a rolled loop over the nodes keeps the executed code small: this code
    // runs once per block, so its instruction fetch is on the critical path)
    bool any = true;
#pragma unroll 1
    for (int j = kNodes - 1; j >= 0 && any; --j) {
      const double xj = s_gx[j];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const double y = gh_point(gp.a, mm[u], sg[u], xj);
        act[u] = act[u] && y > lo;
        if (act[u]) {
          int b = (int)((y - lo) * iw);
          b = b < 0 ? 0 : (b > kNB - 1 ? kNB - 1 : b);
          atomicAdd(&hc[j * kNB + b], nn[u]);
        }
      }
      any = __any(act[0] || act[1] || act[2] || act[3]);
    }
  }
  __syncthreads();
  EKV_MARK(1, 2);
  // the row's counts: integer adds, so the totals do not depend on their order
  unsigned *gc_row = ws.cnt + (size_t)rc.row * kNodes * kNB;
  for (int i = tid; i < kNodes * kNB; i += kGThreads) {
    const unsigned v = hc[i];
    if (v) __hip_atomic_fetch_add(&gc_row[i], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (!arrive_last(&ws.ctr[rc.row * 2 + 0], (unsigned)rc.nch, &s_last)) return;
  EKV_MARK(1, 3);

  // ---- last block of the row: bin weights, edge bounds, window.
  // Bins 2 tid and 2 tid + 1: W_b = sum_j w_j N_bj (fixed order).
  double W[2];
  {
    unsigned long long nv[kNodes];
#pragma unroll
    for (int j = 0; j < kNodes; ++j)
      nv[j] = 2 * tid < kNB ? ld_agent(reinterpret_cast<const unsigned long long *>(gc_row + j * kNB + 2 * tid)) : 0ull;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      double s = 0.0;
#pragma unroll
      for (int j = 0; j < kNodes; ++j) s += gc.w[j] * (double)(unsigned)(nv[j] >> (32 * k));
      W[k] = s;
    }
  }
  // Suffix sums about each bin.  The pair's own suffix about bin 2 tid, then an
  // exclusive suffix scan over the threads above (within the wave by shuffles,
  // the waves above through LDS, each combined in a fixed order).
  const int lane = tid & (kWave - 1), wv = tid / kWave;
  const Z3 pair{W[0] + W[1], W[1], W[1]};
  Z3 x = pair;  // inclusive suffix of this wave's pairs from lane's pair, about bin 2 tid
#pragma unroll
  for (int dist = 1; dist < kWave; dist <<= 1) {
    const double t0 = __shfl_down(x.z0, dist, kWave), t1 = __shfl_down(x.z1, dist, kWave),
                 t2 = __shfl_down(x.z2, dist, kWave);
    if (lane + dist < kWave) x = z_shift_add(x, Z3{t0, t1, t2}, 2.0 * dist);
  }
  if (lane == 0) s_wave[wv] = x;
  s_w1[tid] = W[1];
  Z3 ex;  // suffix of the bins from 2 tid + 2 on, about bin 2 tid + 2
  {
    const double e0 = __shfl_down(x.z0, 1, kWave), e1 = __shfl_down(x.z1, 1, kWave),
                 e2 = __shfl_down(x.z2, 1, kWave);
    ex = lane + 1 < kWave ? Z3{e0, e1, e2} : Z3{0.0, 0.0, 0.0};
  }
  __syncthreads();
  {
    Z3 up{0.0, 0.0, 0.0};  // the waves above, about the first bin of wave wv + 1
    for (int v = kGThreads / kWave - 1; v > wv; --v) up = z_shift_add(s_wave[v], up, 2.0 * kWave);
    ex = z_shift_add(ex, up, 2.0 * (kWave - 1 - lane));
  }
  const Z3 zb0 = z_shift_add(pair, ex, 2.0);                  // from bin 2 tid
  const Z3 zb1 = z_shift_add(Z3{W[1], 0.0, 0.0}, ex, 1.0);    // from bin 2 tid + 1
  const Z3 zbm = z_shift_add(Z3{tid > 0 ? s_w1[tid - 1] : 0.0, 0.0, 0.0}, zb0, 1.0);  // from bin 2 tid - 1
  // A point counted in bin b' was placed by one rounding of (y - lo) / w, so it
  // lies in [e_b'-1, e_b'+2).  Hence, with Z_r(c) = sum_{b' >= c} (b' - c)^r W_b'
  // and e_b' - e_b = (b' - b) w:
  //   F(e_b) >= LB(e_b) = w^beta Z_beta(b + 1),
  //   F(e_b) <= UB(e_b) = w^beta sum_{m >= 0} W_{b-1+m} (m + 1)^beta
  //                     = w^beta [Z_2 + 2 Z_1 + Z_0](b - 1)   (beta 2)
  //                     = w^beta [Z_1 + Z_0](b - 1)           (beta 1).
  // The edges carry rounding errors of about 1e-16 max(|lo|, |hi|), negligible
  // against kCertEps unless the bins are narrower than 1e-6 of that: then the
  // window is the whole range (the solve below is exact on any window).
  const bool resolved = w >= 1e-6 * fmax(fabs(lo), fabs(hi));
  const double wb = gp.ibeta == 2 ? w * w : w;
  auto lbf = [&](const Z3 &z) { return (gp.ibeta == 2 ? z.z2 : z.z1) * wb; };
  auto ubf = [&](const Z3 &z) { return (gp.ibeta == 2 ? z.z2 + 2.0 * z.z1 + z.z0 : z.z1 + z.z0) * wb; };
  int klo = 0, khi = kNB;
  if (2 * tid < kNB) {
    if (lbf(zb1) >= 1.0 + kCertEps) klo = 2 * tid;      // edge 2 tid
    if (lbf(ex) >= 1.0 + kCertEps) klo = 2 * tid + 1;   // edge 2 tid + 1
    if (ubf(zb0) < 1.0 - kCertEps) khi = 2 * tid + 1;
    if (ubf(zbm) < 1.0 - kCertEps) khi = 2 * tid;
  }
  if (tid == 0) { s_klo = 0; s_khi = kNB; }
  __syncthreads();
  if (klo > 0) atomicMax(&s_klo, klo);
  if (khi < kNB) atomicMin(&s_khi, khi);
  __syncthreads();
  if (tid == 0) {
    int a = s_klo, b = s_khi;
    if (!resolved || !(b > a)) { a = 0; b = kNB; }  // (b > a holds for certified bounds)
    ws.win[rc.row * 2 + 0] = a;
    ws.win[rc.row * 2 + 1] = b;
  }
  EKV_MARK(1, 4);
}


// F = 1 on the window [elo, ehi] for rows with at most kWave * kWinReg window
// points, on one wave (no block barriers): Newton from the left, and each pass
// also solves its piece exactly.  With A the window points above t and every
// point above ehi active (moments S about ehi), F(t + u) = f - fp u + q u^2
// (beta 2, q = sum_A c + S0) or f - fp u (beta 1) until u reaches the nearest
// point of A; the smaller root of F(t + u) = 1, when it stays below that point
// and inside the window, is F's root.
__device__ double window_root_wave(const double (&v)[kWinReg], const double (&c)[kWinReg], double elo, double ehi,
                                   double S0, double S1, double S2, int ibeta) {
  double t = elo;
#pragma unroll 1
  for (int it = 0; it < 200; ++it) {
    double f = 0.0, fp = 0.0, qa = 0.0, nmn = -INFINITY;
#pragma unroll
    for (int u = 0; u < kWinReg; ++u) {
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
    const double Dd = ehi - t;  // >= 0
    if (ibeta == 2) { f += S2 + 2.0 * Dd * S1 + Dd * Dd * S0; fp += 2.0 * S1 + 2.0 * Dd * S0; }
    else { f += S1 + Dd * S0; fp += S0; }
    if (!(fp > 0.0)) break;
    if (f > 1.0) {
      const double q = qa + S0;
      const double u = ibeta == 2 ? (f - 1.0) / (0.5 * fp + sqrt(fmax(0.25 * fp * fp - q * (f - 1.0), 0.0)))
                                  : (f - 1.0) / fp;
      if (u <= -nmn && t + u <= ehi) return t + u;
    }
    double tn = t + (f - 1.0) / fp;
    if (tn > ehi) tn = ehi;
    if (!(tn > t)) break;  // converged from the left (or rounding stalls)
    t = tn;
  }
  return t;
}

// Window point k of a row: its code (page * 16 + node) from the chunk
// segments (woff: prefix of the chunks' counts), then its point and weight
// recomputed with the expression the chunk pass used.
struct WinPoints {
  const int *seg;    // the row's window-point region
  const int *woff;   // LDS, [nch + 1]
  int nch, chunk;
  const float *mu, *var;
  size_t base;
  int L, P;
  double a;
  const GaussConsts *gc;
  __device__ __forceinline__ void get(int k, double &y, double &c) const {
    int lo = 0, hi = nch - 1;  // chunk holding point k
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (woff[mid] <= k) lo = mid; else hi = mid - 1;
    }
    const int code = ld_agent(&seg[(size_t)lo * chunk * kNodes + (k - woff[lo])]);
    const int p = code >> 4, j = code & 15;
    const double sig = sigma_of(var[base + p]);
    y = gh_point(a, (double)mu[base + p], sig, gc->x[j]);
    c = (double)min(P, L - p * P) * gc->w[j];
  }
};

// ------------------------------------------------------------------ K3: solve
__global__ __launch_bounds__(kGThreads) void gauss_solve_kernel(
    Dims D, GaussParams gp, GaussConsts gc, const float *__restrict__ box, const float *__restrict__ mu,
    const float *__restrict__ var, const int32_t *__restrict__ seq_lens, const uint8_t *__restrict__ seq_mask,
    int32_t *__restrict__ sel_idx, int32_t *__restrict__ sel_cnt, double *__restrict__ tau_hat, GaussWs ws) {
  __shared__ int scan_scratch[kGThreads / kWave];
  __shared__ double dred[3 * kGThreads / kWave];
  __shared__ int s_last, s_best_p;
  __shared__ int s_off[kMaxChunks + 1], s_woff[kMaxChunks + 1];
  __shared__ double s_ae[kMaxChunks];
  __shared__ int s_ap[kMaxChunks];
  __shared__ double s_tau;
  __shared__ double s_red[2 * kGThreads / kWave];
  __shared__ double s_wy[kWave * kWinReg], s_wc[kWave * kWinReg];
  __shared__ double s_gx[kNodes], s_gw[kNodes];
  const RowChunk bc = map_block(blockIdx.x, gp);
  if (!bc.ok) return;
  EKV_MARK(2, 0);
  const RowCtx rc = row_ctx(D, gp, seq_lens, seq_mask, bc.row);
  if (!rc.active) return;
  const int tid = threadIdx.x, chunk = bc.chunk;
  const size_t base = (size_t)rc.row * D.max_pages;
  const int p_begin = chunk * gp.chunk, p_end = min(rc.np, p_begin + gp.chunk);
  // independent loads first: this chunk's first pages, the window, the bracket
  Pages4 pg0;
  if (chunk < rc.nch) pg0.load(box, mu, var, base, p_begin + 4 * tid, D, gp);
  if (tid < kNodes) {  // read in the node loop below (ordered by row_bracket's barrier)
    s_gx[tid] = gc.x[tid];
    s_gw[tid] = gc.w[tid];
  }
  const int klo = ws.win[rc.row * 2 + 0], khi = ws.win[rc.row * 2 + 1];
  double lo, hi;
  row_bracket(D, gp, ws, rc, box, mu, var, lo, hi, s_red);
  if (!(hi > -INFINITY)) {  // no pages, or none valid: empty selection
    if (chunk == 0 && tid == 0) {
      sel_cnt[rc.row] = 0;
      if (tau_hat) tau_hat[rc.row] = NAN;
    }
    return;
  }
  if (chunk >= rc.nch) return;
  EKV_MARK(2, 1);
  const double w = (hi - lo) / kNB;
  const double elo = edge(lo, hi, w, klo), ehi = edge(lo, hi, w, khi);
  const double thr_lo = elo / gp.a - gp.delta, thr_hi = ehi / gp.a - gp.delta;
  int *wseg = ws.wpts + (size_t)rc.row * D.max_pages * kNodes + (size_t)chunk * gp.chunk * kNodes;

  // ---- per thread, in a fixed order (groups, then nodes from the top, then
  // the thread's 4 pages): moments of the points above ehi about ehi, the
  // window points, the page codes and the largest estimate
  double S[3] = {0.0, 0.0, 0.0};
  double Su[4][3] = {{0.0, 0.0, 0.0}, {0.0, 0.0, 0.0}, {0.0, 0.0, 0.0}, {0.0, 0.0, 0.0}};
  int listed = 0, wlisted = 0;
  double best = -INFINITY;
  int bestp = 0x7FFFFFFF;
#pragma unroll 1
  for (int p0 = p_begin + 4 * tid; p0 - 4 * tid < p_end; p0 += kGroup) {
    Pages4 pg = pg0;
    if (p0 != p_begin + 4 * tid) pg.load(box, mu, var, base, p0, D, gp);
    double mm[4], sg[4], nn[4];
    bool act[4];
    int code[4];
    unsigned wm[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = p0 + u;
      const bool valid = p < p_end && page_valid(pg.bx[u], pg.m[u], pg.v2[u]);
      act[u] = valid;
      wm[u] = 0u;
      mm[u] = (double)pg.m[u];
      const double s2d = pg.v2[u] > 0.0f ? (double)pg.v2[u] : 0.0;
      sg[u] = sqrt(s2d);
      nn[u] = (double)max(0, min(D.P, rc.L - p * D.P));
      code[u] = -1;
      if (valid) {
        if (keep_at(thr_hi, pg.bx[u], pg.m[u], s2d, gp.nsig)) code[u] = p;
        else if (keep_at(thr_lo, pg.bx[u], pg.m[u], s2d, gp.nsig)) code[u] = p | (int)0x80000000;
        const double e1 = mm[u] + gp.nsig * sg[u];
        const double est = e1 < (double)pg.bx[u] ? e1 : (double)pg.bx[u];
        if (est > best || (est == best && p < bestp)) { best = est; bestp = p; }
      }
    }
    // branch-free: a point at or below e_hi adds zeros; each of the 4 pages
    // keeps its own moment sums (independent chains), combined in page order
    // after the loop
    bool any = true;
#pragma unroll 1
    for (int j = kNodes - 1; j >= 0 && any; --j) {
      const double xj = s_gx[j], wj = s_gw[j];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const double y = gh_point(gp.a, mm[u], sg[u], xj);
        const bool up = act[u] && y > ehi;
        const double c = up ? nn[u] * wj : 0.0, d = up ? y - ehi : 0.0;
        Su[u][0] += c;
        Su[u][1] += c * d;
        if (gp.ibeta == 2) Su[u][2] += c * d * d;
        wm[u] |= (act[u] && !up && y > elo) ? 1u << j : 0u;
        act[u] = act[u] && y > elo;
      }
      any = __any(act[0] || act[1] || act[2] || act[3]);
    }
    // window points and page codes of this group, in page order: one scan of
    // both counts packed in one word (each below 2^16 per group)
    const int mw = __popc(wm[0]) + __popc(wm[1]) + __popc(wm[2]) + __popc(wm[3]);
    const int ml = (code[0] != -1) + (code[1] != -1) + (code[2] != -1) + (code[3] != -1);
    int tot;
    const int pre = block_excl_scan((mw << 16) | ml, scan_scratch, &tot);
    int at = wlisted + (pre >> 16);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      unsigned m = wm[u];
      while (m) {
        const int j = 31 - __clz(m);  // nodes from the top
        m &= ~(1u << j);
        st_agent(&wseg[at++], (p0 + u) * kNodes + j);
      }
    }
    wlisted += tot >> 16;
    at = listed + (pre & 0xFFFF);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (code[u] != -1) st_agent(&ws.list[base + p_begin + at++], code[u]);
    listed += tot & 0xFFFF;
  }
  EKV_MARK(2, 2);
#pragma unroll
  for (int k = 0; k < 3; ++k) S[k] = ((Su[0][k] + Su[1][k]) + Su[2][k]) + Su[3][k];
  block_sum_n<3>(S, dred);
  {
    const double bm = block_max(best, dred);
    if (tid == 0) s_best_p = 0x7FFFFFFF;
    __syncthreads();
    if (best == bm && bestp != 0x7FFFFFFF) atomicMin(&s_best_p, bestp);
    __syncthreads();
    if (tid == 0) {
      const size_t o = (size_t)rc.row * gp.nchunk + chunk;
      st_agent(&ws.mom[o * 3 + 0], S[0]);
      st_agent(&ws.mom[o * 3 + 1], S[1]);
      st_agent(&ws.mom[o * 3 + 2], S[2]);
      st_agent(&ws.wcnt[o], wlisted);
      st_agent(&ws.lcnt[o], listed);
      st_agent(&ws.amax[o * 2 + 0], bm);
      st_agent(&ws.amax[o * 2 + 1], (double)s_best_p);
    }
  }
  if (!arrive_last(&ws.ctr[rc.row * 2 + 1], (unsigned)rc.nch, &s_last)) return;
  EKV_MARK(2, 3);

  // ---- last block of the row: chunk partials (counts and offsets by block
  // scans, moments summed in chunk order), then the solve on the window
  const int nch = rc.nch;
  {
    // every chunk's partials requested at once (chunk c by thread c mod 256),
    // counts staged in LDS, moments summed in a fixed order
    double sm[3] = {0.0, 0.0, 0.0};
    for (int c = tid; c < nch; c += kGThreads) {
      const size_t o = (size_t)rc.row * gp.nchunk + c;
      const int lc = ld_agent(&ws.lcnt[o]), wc = ld_agent(&ws.wcnt[o]);
      const double ae = ld_agent(&ws.amax[o * 2 + 0]), ap = ld_agent(&ws.amax[o * 2 + 1]);
      const double m0 = ld_agent(&ws.mom[o * 3 + 0]), m1 = ld_agent(&ws.mom[o * 3 + 1]),
                   m2 = ld_agent(&ws.mom[o * 3 + 2]);
      s_off[c + 1] = lc;
      s_woff[c + 1] = wc;
      s_ae[c] = ae;
      s_ap[c] = (int)ap;
      sm[0] += m0;
      sm[1] += m1;
      sm[2] += m2;
    }
    block_sum_n<3>(sm, dred);
    S[0] = sm[0];
    S[1] = sm[1];
    S[2] = sm[2];
    // offsets: thread t owns chunk slots 4t .. 4t + 3 (kMaxChunks = 4 kGThreads)
    static_assert(kMaxChunks == 4 * kGThreads, "four chunk slots per thread");
    int lc[4], wc[4], ls = 0, wsum = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = 4 * tid + u;
      lc[u] = c < nch ? s_off[c + 1] : 0;
      wc[u] = c < nch ? s_woff[c + 1] : 0;
      ls += lc[u];
      wsum += wc[u];
    }
    int ltot, wtot;
    const int pre = block_excl_scan(ls, scan_scratch, &ltot);
    const int wpre = block_excl_scan(wsum, scan_scratch, &wtot);
    __syncthreads();
    int lrun = pre, wrun = wpre;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = 4 * tid + u;
      if (c < nch) {
        s_off[c] = lrun;
        s_woff[c] = wrun;
      }
      lrun += lc[u];
      wrun += wc[u];
    }
    if (tid == 0) {
      s_off[nch] = ltot;
      s_woff[nch] = wtot;
    }
  }
  __syncthreads();
  const int nw = s_woff[nch], n_listed = s_off[nch];
  const WinPoints wp{ws.wpts + (size_t)rc.row * D.max_pages * kNodes, s_woff, nch, gp.chunk, mu, var, base,
                     rc.L, D.P, gp.a, &gc};
  EKV_MARK(2, 4);
  // The list entries (up to kLReg per thread, with the statistics of the
  // undecided ones) and, for the one-wave solve, the window points are all
  // requested before anything waits: two dependent rounds of loads in all.
  constexpr int kLReg = 4;
  const bool wave_solve = nw <= kWave * kWinReg;
  int lcode[kLReg];
  float lbx[kLReg], lmu[kLReg], lva[kLReg];
  auto list_at = [&](int e) {
    int lo_c = 0, hi_c = nch - 1;  // chunk holding entry e
    while (lo_c < hi_c) {
      const int mid = (lo_c + hi_c + 1) >> 1;
      if (s_off[mid] <= e) lo_c = mid; else hi_c = mid - 1;
    }
    return ld_agent(&ws.list[base + (size_t)lo_c * gp.chunk + (e - s_off[lo_c])]);
  };
#pragma unroll
  for (int u = 0; u < kLReg; ++u) {
    const int e = u * kGThreads + tid;
    lcode[u] = e < n_listed ? list_at(e) : 0;
  }
  if (wave_solve) {
#pragma unroll
    for (int u = 0; u < (kWave * kWinReg) / kGThreads; ++u) {
      const int k = u * kGThreads + tid;
      double y = -INFINITY, c = 0.0;
      if (k < nw) wp.get(k, y, c);
      s_wy[k] = y;
      s_wc[k] = c;
    }
  }
#pragma unroll
  for (int u = 0; u < kLReg; ++u) {
    const int e = u * kGThreads + tid;
    const int p = lcode[u] & 0x7FFFFFFF;
    lbx[u] = lmu[u] = lva[u] = 0.0f;
    if (e < n_listed && lcode[u] < 0) {
      lbx[u] = box[base + p];
      lmu[u] = mu[base + p];
      lva[u] = var[base + p];
    }
  }
  __syncthreads();
  double t = elo;
  if (wave_solve) {
    if (tid < kWave) {
      double wv[kWinReg], wcw[kWinReg];
#pragma unroll
      for (int u = 0; u < kWinReg; ++u) {
        wv[u] = s_wy[u * kWave + tid];
        wcw[u] = s_wc[u * kWave + tid];
      }
      const double tw = window_root_wave(wv, wcw, elo, ehi, S[0], S[1], S[2], gp.ibeta);
      if (tid == 0) s_tau = tw;
    }
    __syncthreads();
    t = s_tau;
  } else {
    // many window points: kBlkReg per thread in registers, the rest recomputed per pass
    double rv[kBlkReg], rcw[kBlkReg];
#pragma unroll
    for (int u = 0; u < kBlkReg; ++u) {
      const int k = u * kGThreads + tid;
      double y = -INFINITY, c = 0.0;
      if (k < nw) wp.get(k, y, c);
      rv[u] = y;
      rcw[u] = c;
    }
#pragma unroll 1
    for (int it = 0; it < 200; ++it) {
      double sm[3] = {0.0, 0.0, 0.0};  // f, fp, sum_A c over the window points
      double nmn = -INFINITY;
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
      for (int u = 0; u < kBlkReg; ++u) acc_pt(rv[u], rcw[u]);
      for (int k = kBlkReg * kGThreads + tid; k < nw; k += kGThreads) {
        double y, c;
        wp.get(k, y, c);
        acc_pt(y, c);
      }
      block_sum_n<3>(sm, dred);
      nmn = block_max(nmn, dred);
      double f = sm[0], fp = sm[1];
      const double Dd = ehi - t;
      if (gp.ibeta == 2) { f += S[2] + 2.0 * Dd * S[1] + Dd * Dd * S[0]; fp += 2.0 * S[1] + 2.0 * Dd * S[0]; }
      else { f += S[1] + Dd * S[0]; fp += S[0]; }
      if (!(fp > 0.0)) break;
      if (f > 1.0) {
        const double q = sm[2] + S[0];
        const double u = gp.ibeta == 2 ? (f - 1.0) / (0.5 * fp + sqrt(fmax(0.25 * fp * fp - q * (f - 1.0), 0.0)))
                                       : (f - 1.0) / fp;
        if (u <= -nmn && t + u <= ehi) {
          t = t + u;
          break;
        }
      }
      double tn = t + (f - 1.0) / fp;
      if (tn > ehi) tn = ehi;
      if (!(tn > t)) break;
      t = tn;
    }
  }
  EKV_MARK(2, 5);
  if (tid == 0 && tau_hat) tau_hat[rc.row] = t / gp.a;
  const double thr = t / gp.a - gp.delta;

  // ---- settle the undecided pages and write the ascending list (the first
  // kLReg * kGThreads entries from registers, any further ones loaded here)
  int total = 0;
  for (int e0 = 0; e0 < n_listed; e0 += kGThreads) {
    const int e = e0 + tid, u = e0 / kGThreads;
    int take = 0, p = 0;
    if (e < n_listed) {
      int code;
      float bx, m, v2;
      if (u < kLReg) {
        code = lcode[0];
#pragma unroll
        for (int k = 1; k < kLReg; ++k)
          if (u == k) code = lcode[k];
        bx = lbx[0]; m = lmu[0]; v2 = lva[0];
#pragma unroll
        for (int k = 1; k < kLReg; ++k)
          if (u == k) { bx = lbx[k]; m = lmu[k]; v2 = lva[k]; }
      } else {
        code = list_at(e);
        const int q = code & 0x7FFFFFFF;
        bx = box[base + q]; m = mu[base + q]; v2 = var[base + q];
      }
      p = code & 0x7FFFFFFF;
      if (code >= 0) take = 1;
      else take = keep_at(thr, (double)bx, (double)m, v2 > 0.0f ? (double)v2 : 0.0, gp.nsig) ? 1 : 0;
    }
    int tot;
    const int pos = block_excl_scan(take, scan_scratch, &tot);
    if (take) sel_idx[base + total + pos] = p;
    total += tot;
  }
  if (tid == 0) {
    if (total == 0) {  // nothing kept: the page of largest estimate, lowest index on ties
      double be = -INFINITY;
      int bp = 0x7FFFFFFF;
      for (int c = 0; c < nch; ++c) {
        if (s_ap[c] == 0x7FFFFFFF) continue;
        if (bp == 0x7FFFFFFF || s_ae[c] > be) { be = s_ae[c]; bp = s_ap[c]; }
      }
      sel_idx[base] = bp;
      total = 1;
    }
    sel_cnt[rc.row] = total;
  }
  EKV_MARK(2, 6);
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
  gp.lone_full = gp.ibeta == 2 ? std::sqrt(2.5 / (double)D.P) : 2.5 / (double)D.P;
  gp.rows = D.B * D.Hq;
  gp.vec = 0;
  gp.sum_tiles = 0;
  // about EKV_GAUSS_BLOCKS blocks over the (row, chunk) space; chunks are
  // multiples of 256 pages (4 per thread of one 1024-page group), at most
  // kMaxChunks per row
  const int want = (EKV_GAUSS_BLOCKS + gp.rows - 1) / gp.rows;
  int chunk = (D.max_pages + want - 1) / want;
  chunk = ((chunk + 255) / 256) * 256;
  if (chunk > kGroup) chunk = ((chunk + kGroup - 1) / kGroup) * kGroup;
  if (chunk < 256) chunk = 256;
  if ((D.max_pages + chunk - 1) / chunk > kMaxChunks)
    chunk = (((D.max_pages + kMaxChunks - 1) / kMaxChunks + kGroup - 1) / kGroup) * kGroup;
  gp.chunk = chunk;
  gp.nchunk = (D.max_pages + chunk - 1) / chunk;
  return gp;
}

static GaussWs carve_gauss(const Dims &D, const GaussParams &gp, void *base, size_t *bytes) {
  Carve cv(base);
  const size_t rows = (size_t)D.B * D.Hq;
  GaussWs w;
  w.cnt = cv.take<unsigned>(rows * kNodes * kNB);  // counts and counters first: one zeroed range
  w.ctr = cv.take<unsigned int>(rows * 2);
  w.part = cv.take<double>(rows * gp.nchunk * 2);
  w.summ = nullptr;
  w.win = cv.take<int>(rows * 2);
  w.mom = cv.take<double>(rows * gp.nchunk * 3);
  w.wcnt = cv.take<int>(rows * gp.nchunk);
  w.wpts = cv.take<int>(rows * (size_t)D.max_pages * kNodes);
  w.list = cv.take<int>(rows * (size_t)D.max_pages);
  w.lcnt = cv.take<int>(rows * gp.nchunk);
  w.amax = cv.take<double>(rows * gp.nchunk * 2);
  if (bytes) *bytes = cv.bytes();
  return w;
}

size_t gauss_ws_bytes(const Dims &D) {
  GaussParams gp = make_params(D, 1.5, 0.0, 3.0);
  size_t bytes = 0;
  carve_gauss(D, gp, nullptr, &bytes);
  return bytes;
}

static hipError_t launch_gauss_impl(const Dims &D, const float *box, const float *mu, const float *var,
                                    const int32_t *seq_lens, double alpha, double delta, double n_sigma,
                                    const uint8_t *seq_mask, int32_t *sel_idx, int32_t *sel_cnt,
                                    double *tau_hat, const double *summ, void *ws, hipStream_t s) {
  GaussParams gp = make_params(D, alpha, delta, n_sigma);
  const GaussConsts &gc = gauss_consts();
  const int rows = D.B * D.Hq;
  if (gp.ibeta == 0) {
    hipLaunchKernelGGL(gauss_generic_kernel, dim3(rows), dim3(kGenThreads), 0, s, D, gp, gc, box, mu,
                       var, seq_lens, seq_mask, sel_idx, sel_cnt, tau_hat);
    return hipGetLastError();
  }
  const uintptr_t al = reinterpret_cast<uintptr_t>(box) | reinterpret_cast<uintptr_t>(mu) |
                       reinterpret_cast<uintptr_t>(var);
  gp.vec = (al % 16 == 0 && D.max_pages % 4 == 0) ? 1 : 0;
  GaussWs w = carve_gauss(D, gp, ws, nullptr);
  const dim3 grid(grid_of(gp));
  if (summ) {  // bracket from the scorer's summary; counts and counters zeroed by the scorer
    gp.sum_tiles = (D.max_pages + kSummaryTile - 1) / kSummaryTile;
    w.summ = summ;
  } else {
    hipLaunchKernelGGL(gauss_bracket_kernel, grid, dim3(kGThreads), 0, s, D, gp, gc, box, mu, var, seq_lens,
                       seq_mask, w);
  }
  hipLaunchKernelGGL(gauss_count_kernel, grid, dim3(kGThreads), 0, s, D, gp, gc, box, mu, var, seq_lens,
                     seq_mask, w);
  hipLaunchKernelGGL(gauss_solve_kernel, grid, dim3(kGThreads), 0, s, D, gp, gc, box, mu, var, seq_lens,
                     seq_mask, sel_idx, sel_cnt, tau_hat, w);
  return hipGetLastError();
}

hipError_t launch_gauss(const Dims &D, const float *box, const float *mu, const float *var,
                        const int32_t *seq_lens, double alpha, double delta, double n_sigma,
                        const uint8_t *seq_mask, int32_t *sel_idx, int32_t *sel_cnt,
                        double *tau_hat, void *ws, hipStream_t s) {
  return launch_gauss_impl(D, box, mu, var, seq_lens, alpha, delta, n_sigma, seq_mask, sel_idx, sel_cnt, tau_hat,
                           nullptr, ws, s);
}

hipError_t launch_gauss_from_summary(const Dims &D, const float *box, const float *mu, const float *var,
                                     const int32_t *seq_lens, double alpha, double delta, double n_sigma,
                                     const uint8_t *seq_mask, int32_t *sel_idx, int32_t *sel_cnt,
                                     double *tau_hat, const double *summ, void *ws, hipStream_t s) {
  return launch_gauss_impl(D, box, mu, var, seq_lens, alpha, delta, n_sigma, seq_mask, sel_idx, sel_cnt, tau_hat,
                           summ, ws, s);
}

long long gauss_zero_words(const Dims &D, void *ws, unsigned **zero) {
  *zero = static_cast<unsigned *>(ws);
  return (long long)D.B * D.Hq * (kNodes * kNB + 2);
}

EKV_TRACE_DUMP(ekv_trace_dump_gauss)
}  // namespace ekv
