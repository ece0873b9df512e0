// decode_items.hip -- alpha-entmax attention over selected pages, per item
// ([EntmaxKV s.2.C]): the decode for a few query-head rows (single-sequence
// decode), where the time is latency, not bandwidth.
//
// EntmaxKV s.2.C = section 2.C ("sparse entmax attention") of "Resumen Tecnico:
// EntmaxKV - Decodificacion Consciente del Soporte para Atencion Entmax",
// gist.science/es/paper/2605.21649: load only the KV entries of the selected
// pages and compute the alpha-entmax weights over that reduced set.
//
// alpha-entmax (Peters, Niculae & Martins 2019): with X_t = (alpha-1) s_t,
// p_t = [X_t - tau]_+^(1/(alpha-1)), tau the root of sum_t p_t = 1.
//
// Two launches.
//  1. Scores.  Work is a flat list of items (row, i): the i-th selected page of
//     query row (b, h), strided over a fixed grid so that every kept page's K
//     slice is requested at once; every block maps items through a prefix sum
//     of the selection counts it computes itself.  An item writes the exact fp64
//     scores X of the page's tokens (bf16 products are exact; fp64 sums), the
//     page's maximum (NaN for a malformed item) and its physical page, at the
//     row's first item plus i (rows past the workspace's capacity are skipped).
//  2. Threshold and output.  Since F(max X - 1) >= 1, tau is at least
//     max X - 1 and only tokens with X > max X - 1 can carry weight.  Each row
//     is cut into up to kSplitMax chunks of kChunkTok tokens; the block of a
//     chunk reads the row's page maxima, compacts its chunk's candidates in
//     place, and the row's last block (atomic handshake; kernel 1 zeroed the
//     counters) gathers them into LDS.  tau comes from safeguarded Newton from
//     the left on the candidates (one wave and shuffles when they are few) or
//     from the sparsemax sort form; the V rows of the support are then
//     gathered with 16-byte loads.  Kept tokens outside the support cost no V
//     traffic.  Rows with more candidates than LDS holds are solved by passes
//     over the compacted candidates in the workspace.
//
// A kept page is scored once per query head here (a group's heads rarely keep
// the same pages when a few pages per head are kept); the decode for many rows
// (decode.hip) scores each page once per KV head.
#include <math.h>

#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace ekv {
namespace items {

constexpr int kDThreads = 256;
constexpr int kDGrid = 2048;      // kernel 1: items are strided over this many blocks
constexpr int kChunkTok = 2048;   // kernel 2: tokens per chunk block (long_1m decode: 2048 26.6 us, 1024 30.3, 4096 27.2, 8192 30.9)
constexpr int kSplitMax = 32;     // kernel 2: chunk blocks per row at most
constexpr int kCand = 1024;       // candidates a last block keeps in LDS (one wave solves for tau)
constexpr int kSupChunk = 512;    // support entries gathered per LDS pass
constexpr int kNThr = 8;          // count thresholds mx - 2^-i behind the certified bound on tau
constexpr int kKeepIt = 3;        // kernel 2: 2048-token steps of a chunk kept in registers between passes
constexpr int kIprLds = 2048;     // kernel 2: a split row's item -> physical page table staged in LDS up to this size

struct DecodeWs {
  double *xs;        // [cap*P]  X of kept tokens, item-major (row r's item i at rbase[r] + i);
                     //          kernel 2 compacts each chunk's candidates to the chunk's start
  uint32_t *xi;      // [cap*P]  token index (item*P + slot) of a compacted candidate
  double *pmax;      // [cap]    max X over an item's tokens, NaN if the item is malformed
  uint32_t *iphys;   // [cap]    physical page of an item
  long long *rbase;  // [rows]   first item of each row (written by kernel 1)
  long long cap;     //          items the workspace holds; rows past it read NaN
  int *segcnt;       // [rows][kSplitMax]    candidates of each chunk
  double *segL;      // [rows][kSplitMax]    each chunk's lower bound on tau
  int *segn;         // [rows][kSplitMax][kNThr] each chunk's counts above mx - 2^-i
  unsigned int *ctr; // [rows]               arrival counters (zeroed by kernel 1)
};

struct DecodeParams {
  double a, beta, c;
  int ibeta, tau_method;
};

// pow for the generic exponent, kept out of line: the solver loops are
// unrolled and would otherwise carry one copy per call site.
__device__ __noinline__ double pow_generic(double x, double y) { return pow(x, y); }

__device__ __forceinline__ double pw_rt(double x, const DecodeParams &dp) {
  return dp.ibeta == 2 ? x * x : (dp.ibeta == 1 ? x : pow_generic(x, dp.beta));
}

// c^-(alpha-1)
__device__ __forceinline__ double pow_neg_a(double c, const DecodeParams &dp) {
  return dp.ibeta == 2 ? 1.0 / sqrt(c) : (dp.ibeta == 1 ? 1.0 / c : pow_generic(c, -dp.a));
}

// The same powers with the exponent fixed at compile time (kB = 2: alpha = 1.5,
// kB = 1: alpha = 2, kB = 0: any alpha through pow).
template <int kB>
__device__ __forceinline__ double pw(double y, const DecodeParams &dp) {
  if constexpr (kB == 2) return y * y;
  else if constexpr (kB == 1) return y;
  else return pow_generic(y, dp.beta);
}
template <int kB>
__device__ __forceinline__ double pw_d(double y, const DecodeParams &dp) {
  if constexpr (kB == 2) return 2.0 * y;
  else if constexpr (kB == 1) return 1.0;
  else return dp.beta * pow_generic(y, dp.beta - 1.0);
}

// Selected-page count of a row clamped to [0, max_pages]; *bad is set for a
// count outside [0, number of pages of the sequence].
__device__ __forceinline__ int row_items(const Dims &D, const int32_t *seq_lens, const int32_t *sel_cnt,
                                         int row, bool *bad) {
  const int np = n_pages_of(seq_len_clamped(seq_lens, row / D.Hq, D), D.P);
  int c = sel_cnt[row];
  *bad = c < 0 || c > np;
  return c < 0 ? 0 : (c > D.max_pages ? D.max_pages : c);
}

// Block-shared item map: prefix[r] = first item of row r, prefix[rows] = total.
// Each thread owns a contiguous run of rows; its counts are loaded 8 at a time.
__device__ int build_item_map(const Dims &D, const int32_t *seq_lens, const int32_t *sel_cnt,
                              int *prefix, int rows, int *scan_scratch) {
  const int per = (rows + kDThreads - 1) / kDThreads;
  const int r0 = threadIdx.x * per;
  int sum = 0;
#pragma unroll 1
  for (int c0 = 0; c0 < per; c0 += 8) {
    int c[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      bool bad;
      c[u] = row_items(D, seq_lens, sel_cnt, min(r0 + c0 + u, rows - 1), &bad);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = r0 + c0 + u;
      if (c0 + u < per && r < rows) { prefix[r] = c[u]; sum += c[u]; }
    }
  }
  int tot;
  int run = block_excl_scan(sum, scan_scratch, &tot);
#pragma unroll 1
  for (int u = 0; u < per; ++u) {
    const int r = r0 + u;
    if (r < rows) { const int c = prefix[r]; prefix[r] = run; run += c; }
  }
  if (threadIdx.x == 0) prefix[rows] = tot;
  __syncthreads();
  return tot;
}
__device__ __forceinline__ int find_row(const int *prefix, int rows, int item) {
  int lo = 0, hi = rows - 1;  // largest r with prefix[r] <= item
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= item) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ------------------------------------------------------------- threshold solve
// Values seen by the solver: LDS candidates (strided over the participating
// threads) or, for a row whose candidates overflow LDS, every score of the row
// in the workspace above the bound `thr` (batched agent-scope loads).
struct LdsVals {
  const double *v;
  int n, t0, stride;
  template <typename Fn>
  __device__ __forceinline__ void each(Fn &&fn) const {
#pragma unroll 2
    for (int i = t0; i < n; i += stride) fn(v[i]);
  }
};
// Compacted candidates in the workspace: segment s (chunk s of the row) holds
// soff[s+1]-soff[s] entries from token offset sbase[s]; entry k of the
// concatenation is found by a scan over the (at most kSplitMax) segments.
template <int kBatch>
struct GlobSeg {
  const double *x;
  const int *soff;   // LDS, [nseg + 1] first entry of each segment
  const int *sbase;  // LDS, [nseg]     token offset where each segment starts
  int nseg, n;
  __device__ __forceinline__ int seg_of(int k) const {
    int lo = 0, hi = nseg - 1;  // last segment starting at or before k
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (soff[mid] <= k) lo = mid; else hi = mid - 1;
    }
    return lo;
  }
  __device__ __forceinline__ int addr(int k) const {
    const int lo = seg_of(k);
    return sbase[lo] + (k - soff[lo]);
  }
  // addresses of entries min(k0 + u, n - 1), u < R: one search, then the
  // segment advances with k (empty segments are stepped over)
  template <int R>
  __device__ __forceinline__ void addr_run(int k0, int (&a)[R]) const {
    int lo = seg_of(min(k0, n - 1));
    int next = lo + 1 < nseg ? soff[lo + 1] : 0x7fffffff;
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int k = min(k0 + u, n - 1);
      while (k >= next) {
        ++lo;
        next = lo + 1 < nseg ? soff[lo + 1] : 0x7fffffff;
      }
      a[u] = sbase[lo] + (k - soff[lo]);
    }
  }
  template <typename Fn>
  __device__ __forceinline__ void each(Fn &&fn) const {
#pragma unroll 1
    for (int base = 0; base < n; base += kBatch * kDThreads) {
      double v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) v[u] = ld_agent(&x[addr(min(base + u * kDThreads + (int)threadIdx.x, n - 1))]);
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (base + u * kDThreads + (int)threadIdx.x < n) fn(v[u]);
    }
  }
};

// Candidates held in registers: thread t owns entries 16t .. 16t + 15.
constexpr int kRegPer = 16;
struct RegVals {
  const double (&v)[kRegPer];
  int n;
  template <typename Fn>
  __device__ __forceinline__ void each(Fn &&fn) const {
#pragma unroll
    for (int j = 0; j < kRegPer; ++j)
      if ((int)threadIdx.x * kRegPer + j < n) fn(v[j]);
  }
};
struct WaveRed {
  __device__ __forceinline__ double operator()(double v, double *) const { return wave_sum(v); }
  __device__ __forceinline__ void pair(double &a, double &b, double *) const { a = wave_sum(a); b = wave_sum(b); }
  __device__ __forceinline__ void sums3(double (&v)[3], double *) const {
    v[0] = wave_sum(v[0]); v[1] = wave_sum(v[1]); v[2] = wave_sum(v[2]);
  }
  __device__ __forceinline__ double max(double v, double *) const { return wave_max(v); }
};
struct BlockRed {
  __device__ __forceinline__ double operator()(double v, double *s) const { return block_sum(v, s); }
  __device__ __forceinline__ void pair(double &a, double &b, double *s) const { block_sum2(a, b, s); }
  __device__ __forceinline__ void sums3(double (&v)[3], double *s) const { block_sum_n<3>(v, s); }
  __device__ __forceinline__ double max(double v, double *s) const { return block_max(v, s); }
};

// Root of F(t) = sum [X - t]_+^beta = 1 by Newton from the left: lo0 has
// F >= 1 (mx - 1 or a tighter certified bound), hi = mx - n^-(alpha-1) has
// F <= 1 (n >= the number of scores above hi).  For alpha <= 2 (beta >= 1) F is convex and decreasing, so every
// Newton iterate from the left stays left of the root: one pass per step.
// Otherwise each Newton candidate is checked with a second pass; one that
// leaves (lo, hi) becomes a bisection step, and after a step lands right of
// the root the next step bisects.
//
// alpha = 2 and 1.5 (beta = 1, 2): between consecutive scores F is linear or
// quadratic, F(lo + u) = sum_A (y - u)^beta over the active set A = {y = X - lo
// > 0}.  Each pass also solves that piece exactly (u = (S1 - 1)/|A|, or the
// smaller root (S2 - 1)/(S1 + sqrt(S1^2 - |A|(S2 - 1))) of |A| u^2 - 2 S1 u + S2
// = 1); when u <= min_A y every active score stays active at lo + u, so lo + u
// is F's root and the pass ends the search (*z_out = F there, from the same
// sums).  Otherwise the Newton step is taken as above.  Rows end in 1-4 passes
// instead of 5-8.  *z_out = 0 when the search ends another way.
template <int kB, typename Src, typename Red>
__device__ __forceinline__ double newton_tau(const Src &src, double n, double mx, double lo0,
                                             const DecodeParams &dp, double *dred, double *z_out) {
  const Red red;
  double lo = lo0;
  double hi = mx - pow_neg_a(n, dp);
  *z_out = 0.0;
  if (!(hi > lo)) return lo;
  if (kB == 1 || kB == 2) {
#pragma unroll 1
    for (int it = 0; it < 200; ++it) {
      double sm[3] = {0.0, 0.0, 0.0};  // S1, S2, |A| over y = X - lo > 0
      double nmn = -INFINITY;          // -min_A y
      src.each([&](double x) {
        const double y = x - lo;
        if (y > 0.0) { sm[0] += y; sm[1] += y * y; sm[2] += 1.0; nmn = fmax(nmn, -y); }
      });
      red.sums3(sm, dred);
      nmn = red.max(nmn, dred);
      const double s1 = sm[0], s2 = sm[1], c = sm[2];
      const double f = kB == 2 ? s2 : s1;
      if (!(f > 1.0) || !(c > 0.0)) break;  // at the root (to rounding)
      const double u = kB == 2 ? (s2 - 1.0) / (s1 + sqrt(fmax(s1 * s1 - c * (s2 - 1.0), 0.0))) : (s1 - 1.0) / c;
      if (u <= -nmn) {
        *z_out = kB == 2 ? (s2 - 2.0 * u * s1) + c * u * u : s1 - c * u;
        return lo + u;
      }
      const double cand = lo + (f - 1.0) / (kB == 2 ? 2.0 * s1 : c);
      if (!(cand > lo)) break;  // no progress: converged
      if (!(cand < hi)) break;  // only through rounding, next to the root
      lo = cand;
    }
    return lo;
  }
  if (kB != 0 || dp.beta >= 1.0) {
#pragma unroll 1
    for (int it = 0; it < 200; ++it) {
      double f = 0.0, fp = 0.0;
      src.each([&](double x) {
        const double y = x - lo;
        if (y > 0.0) { f += pw<kB>(y, dp); fp += pw_d<kB>(y, dp); }
      });
      red.pair(f, fp, dred);
      if (!(f > 1.0) || !(fp > 0.0)) break;  // at the root (to rounding)
      const double cand = lo + (f - 1.0) / fp;
      if (!(cand > lo)) break;                 // no progress: converged
      if (!(cand < hi)) break;                 // only through rounding, next to the root
      lo = cand;
    }
    return lo;
  }
  bool bisect_next = false;
#pragma unroll 1
  for (int it = 0; it < 400; ++it) {
    double cand;
    if (bisect_next) {
      cand = 0.5 * (lo + hi);
    } else {
      double f = 0.0, fp = 0.0;
      src.each([&](double x) {
        const double y = x - lo;
        if (y > 0.0) { f += pw<kB>(y, dp); fp += pw_d<kB>(y, dp); }
      });
      red.pair(f, fp, dred);
      cand = fp > 0.0 ? lo + (f - 1.0) / fp : 0.5 * (lo + hi);
      if (!(cand > lo) || !(cand < hi)) {
        if (!(cand > lo) && f >= 1.0) break;  // Newton makes no progress: converged
        cand = 0.5 * (lo + hi);
      }
    }
    if (cand == lo || cand == hi) break;
    double f = 0.0;
    src.each([&](double x) {
      const double y = x - cand;
      if (y > 0.0) f += pw<kB>(y, dp);
    });
    f = red(f, dred);
    if (f >= 1.0) { lo = cand; bisect_next = false; }
    else { hi = cand; bisect_next = true; }
  }
  return lo;
}

// sparsemax closed form (Martins & Astudillo 2016) by a bitonic sort in LDS:
// sort z descending; k* = max{k : 1 + k z_(k) > sum_{j<=k} z_(j)};
// tau = (sum_{j<=k*} z_(j) - 1) / k*.  The condition holds exactly for k <= k*.
// Only the candidates are sorted: every score outside them is below tau.
__device__ double sparsemax_tau_sort(const double *cx, int n, double *buf, double *dred, int *s_kstar) {
  int m = 1;
  while (m < n) m <<= 1;
  for (int i = threadIdx.x; i < m; i += kDThreads) buf[i] = i < n ? cx[i] : -INFINITY;
  if (threadIdx.x == 0) *s_kstar = 0;
  __syncthreads();
#pragma unroll 1
  for (int kk = 2; kk <= m; kk <<= 1) {
#pragma unroll 1
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
  double carry = 0.0;
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
#pragma unroll 1
  for (int c0 = 0; c0 < n; c0 += kDThreads) {
    const int k = c0 + threadIdx.x;
    const double z = k < n ? buf[k] : 0.0;
    double x = z;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const double y = __shfl_up(x, o, kWave);
      if (lane >= o) x += y;
    }
    __syncthreads();
    if (lane == kWave - 1) dred[wv] = x;
    __syncthreads();
    double off = carry, tot = 0.0;
    for (int i = 0; i < kDThreads / kWave; ++i) {
      if (i < wv) off += dred[i];
      tot += dred[i];
    }
    if (k < n && 1.0 + (double)(k + 1) * z > off + x) atomicMax(s_kstar, k + 1);
    carry += tot;
  }
  __syncthreads();
  const int ks = *s_kstar > 0 ? *s_kstar : 1;
  double part = 0.0;
  for (int k = threadIdx.x; k < ks; k += kDThreads) part += buf[k];
  part = block_sum(part, dred);
  return (part - 1.0) / (double)ks;
}

// Threshold tau and normalizer z = sum p of a row from its candidates, which
// sit in LDS (tier 0), in registers (tier 1, not for generic alpha) or in the
// workspace (tier 2).
template <int kB>
__device__ __forceinline__ void solve_row(int tier, const DecodeParams &dp, double mx, double lo0, int total, const double *cx,
                                          double *sortbuf, const double (&rx)[kRegPer], const GlobSeg<1> &gs,
                                          double *dred, int *s_kstar, double *s_tau, double &tau, double &z) {
  const int tid = threadIdx.x;
  const GlobSeg<16> gs8{gs.x, gs.soff, gs.sbase, gs.nseg, gs.n};  // 16 scores per thread in flight per step
  double zk = 0.0;  // F at tau when the solver found it from its sums (else 0)
  if (tier == 0 && kB == 1 && dp.tau_method == 1) {
    tau = sparsemax_tau_sort(cx, total, sortbuf, dred, s_kstar);
  } else if (tier == 0) {
    if (tid < kWave) {
      const double t = newton_tau<kB, LdsVals, WaveRed>(LdsVals{cx, total, tid, kWave}, (double)total, mx, lo0, dp,
                                                         dred, &zk);
      if (tid == 0) { s_tau[0] = t; s_tau[1] = zk; }
    }
    __syncthreads();
    tau = s_tau[0];
    zk = s_tau[1];
  } else if (kB != 0 && tier == 1) {
    tau = newton_tau<kB, RegVals, BlockRed>(RegVals{rx, total}, (double)total, mx, lo0, dp, dred, &zk);
  } else if (kB != 0) {
    tau = newton_tau<kB, GlobSeg<16>, BlockRed>(gs8, (double)total, mx, lo0, dp, dred, &zk);
  } else {
    tau = newton_tau<kB, GlobSeg<1>, BlockRed>(gs, (double)total, mx, lo0, dp, dred, &zk);
  }
  if (zk > 0.0) {
    z = zk;
    return;
  }
  double zz = 0.0;
  auto zsum = [&](double x) { const double y = x - tau; if (y > 0.0) zz += pw<kB>(y, dp); };
  if (tier == 0) LdsVals{cx, total, tid, kDThreads}.each(zsum);
  else if (kB != 0 && tier == 1) RegVals{rx, total}.each(zsum);
  else if (kB != 0) gs8.each(zsum);
  else gs.each(zsum);
  z = block_sum(zz, dred);
}

// ---------------------------------------------------------------- kernel 1: scores
template <typename T, int DIM, int P>
__global__ __launch_bounds__(kDThreads) void decode_scores_kernel(
    Dims D, DecodeParams dp, const T *__restrict__ q, const T *__restrict__ k_pool,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ sel_idx, const int32_t *__restrict__ sel_cnt,
    float *__restrict__ weights_out, DecodeWs ws) {
  extern __shared__ __align__(16) unsigned char smem[];
  // A block scores kIPB items (pages) at once, a group of kGT threads each, 4
  // threads per token: one page of 64 tokens per pass, two of 32, four of 16
  // (small pages would otherwise leave most of the block's loads tiny).
  constexpr int kIPB = P >= 64 ? 1 : 64 / P;
  constexpr int kGT = kDThreads / kIPB;  // threads per item
  constexpr int kParts = kGT / P;        // threads per token
  constexpr int kPer = DIM / kParts;     // coordinates per thread
  constexpr int kGW = kGT / kWave;       // waves per item
  static_assert(kParts >= 1 && kGT % kWave == 0 && DIM % kParts == 0, "item groups of whole waves");
  __shared__ double dred[2 * kDThreads / kWave];
  __shared__ int scan_scratch[kDThreads / kWave];
  const int rows = D.B * D.Hq;
  int *prefix = reinterpret_cast<int *>(smem);
  const int tid = threadIdx.x;
  EKV_MARK(0, 0);
  // kernel 2's arrival counters start at zero
  for (int r = blockIdx.x * kDThreads + tid; r < rows; r += gridDim.x * kDThreads) ws.ctr[r] = 0u;
  const int total = build_item_map(D, seq_lens, sel_cnt, prefix, rows, scan_scratch);
  if (blockIdx.x == 0)
    for (int r = tid; r < rows; r += kDThreads) ws.rbase[r] = prefix[r];
  EKV_MARK(0, 1);
  const int MP = D.max_pages;
  const size_t wrow = (size_t)MP * P;
  const int grp = tid / kGT, gtid = tid % kGT;
  const int tok = gtid / kParts, part = gtid % kParts;
  const int wv = tid / kWave, lane = tid & (kWave - 1);
#pragma unroll 1
  for (int item0 = blockIdx.x * kIPB; item0 < total; item0 += gridDim.x * kIPB) {
    // every thread runs the pass (the group maximum below needs whole waves);
    // a group past the last item, or on a row past the workspace's capacity,
    // computes on clamped indices and stores nothing
    const int item = min(item0 + grp, total - 1);
    const bool live = item0 + grp < total;
    const int r = find_row(prefix, rows, item);
    const int i = item - prefix[r];
    const int cnt = prefix[r + 1] - prefix[r];
    const bool fits = (long long)prefix[r + 1] <= ws.cap;  // the row is within the workspace's capacity
    const size_t it = (size_t)prefix[r] + i;
    const int b = r / D.Hq, g = (r % D.Hq) / D.G;
    // independent loads first: sequence length, page ids, the query slice
    const int L = seq_len_clamped(seq_lens, b, D);
    const int p = sel_idx[(size_t)r * MP + i];
    const int prev = i > 0 ? sel_idx[(size_t)r * MP + i - 1] : -1;
    float qv[kPer];
    load_vec<kPer>(q + (size_t)r * DIM + part * kPer, qv);
    const int np = n_pages_of(L, P);
    const int pc = min(max(p, 0), MP - 1);
    const int phys = page_table[(size_t)b * MP + pc];
    const bool bad_item = p < 0 || p >= np || prev >= p || phys < 0 || phys >= D.num_phys;
    const int physc = min(max(phys, 0), D.num_phys - 1);
    const int n = min(P, L - pc * P);
    float kv[kPer];
    load_vec<kPer>(k_pool + (((size_t)physc * D.Hkv + g) * P + tok) * DIM + part * kPer, kv);
    double acc = 0.0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) acc = __builtin_fma((double)kv[e], (double)qv[e], acc);
#pragma unroll
    for (int o = kParts / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, kWave);
    const double x = tok < n ? dp.a * (dp.c * acc) : -INFINITY;
    const bool store = live && fits;
    if (store && part == 0) ws.xs[it * P + tok] = x;
    // the page maximum: the group's waves, combined through LDS when a page spans several
    double pm = wave_max(x);
    if constexpr (kGW > 1) {
      __syncthreads();
      if (lane == 0) dred[wv] = pm;
      __syncthreads();
      pm = dred[grp * kGW];
#pragma unroll
      for (int k = 1; k < kGW; ++k) pm = fmax(pm, dred[grp * kGW + k]);
    }
    if (store && gtid == 0) {
      ws.pmax[it] = bad_item ? NAN : pm;
      ws.iphys[it] = (uint32_t)physc;
    }
    // weights_out: zero every slot of the pages this item covers, (prev, p]
    // (the last item also covers the pages after p); kernel 2 writes the
    // support weights.
    if (weights_out && store && !bad_item) {
      const size_t lo_s = (size_t)(prev + 1) * P;
      const size_t hi_s = (i == cnt - 1) ? wrow : (size_t)(p + 1) * P;
      for (size_t s = lo_s + gtid; s < hi_s; s += kGT) weights_out[(size_t)r * wrow + s] = 0.0f;
    }
  }
  EKV_MARK(0, 2);
}

// ------------------------------------------------ kernel 2: threshold and output
// kB fixes the power's exponent code (2: alpha = 1.5, 1: alpha = 2) at compile
// time: those kernels hold no call of the generic pow, whose calling
// convention costs the kernel SGPR spills and instructions on every phase
// (0.6 us of ~21 at 1M tokens); kB = 0 takes the code from dp.
template <typename T, int DIM, int P, int kB>
__global__ __launch_bounds__(kDThreads) void decode_finish_kernel(
    Dims D, DecodeParams dp_in, const T *__restrict__ v_pool, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ sel_idx, const int32_t *__restrict__ sel_cnt, float *__restrict__ out,
    double *__restrict__ tau_out, float *__restrict__ weights_out, DecodeWs ws) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int kTpe = DIM / 8;           // threads per support entry in the V gather
  constexpr int kEpp = kDThreads / kTpe;  // support entries per gather pass
  __shared__ double dred[3 * kDThreads / kWave];  // up to three block sums at once
  __shared__ int scan_scratch[kDThreads / kWave];
  __shared__ int s_last, s_kstar;
  __shared__ double s_tau[2];
  __shared__ int soff[kSplitMax + 1], sbase[kSplitMax];
  __shared__ double sL[kSplitMax];
  __shared__ int s_cnt[kDThreads / kWave][kNThr];
  __shared__ uint32_t sup_v[kSupChunk];
  __shared__ int sup_i[kSupChunk];
  __shared__ float sup_w[kSupChunk];
  __shared__ float accs[kEpp][DIM + 1];
  __shared__ uint32_t s_ipr[kIprLds];
  double *cx = reinterpret_cast<double *>(smem);              // [kCand] candidate X
  int *ci = reinterpret_cast<int *>(cx + kCand);              // [kCand] token index
  uint32_t *cv = reinterpret_cast<uint32_t *>(ci + kCand);    // [kCand] V row index
  double *sortbuf = reinterpret_cast<double *>(cv + kCand);   // [kCand] (sort form only)
  DecodeParams dp = dp_in;
  if constexpr (kB != 0) dp.ibeta = kB;
  const int r = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
  EKV_MARK(1, 0);
  const int MP = D.max_pages;
  const size_t wrow = (size_t)MP * P;
  const int g = (r % D.Hq) / D.G;
  bool bad;
  const int cnt = row_items(D, seq_lens, sel_cnt, r, &bad);
  if (cnt == 0) {
    if (c == 0) {
      if (tid == 0 && tau_out) tau_out[r] = NAN;
      for (int i = tid; i < DIM; i += kDThreads) out[(size_t)r * DIM + i] = bad ? NAN : 0.0f;
      if (weights_out)
        for (size_t i = tid; i < wrow; i += kDThreads) weights_out[(size_t)r * wrow + i] = 0.0f;
    }
    return;
  }
  const int nX = cnt * P;
  const int nsplit = min((int)gridDim.y, (nX + kChunkTok - 1) / kChunkTok);
  if (c >= nsplit) return;
  const long long rb = ws.rbase[r];
  if (rb + cnt > ws.cap) {  // past the workspace's capacity
    if (c == 0) {
      if (tid == 0 && tau_out) tau_out[r] = NAN;
      for (int i = tid; i < DIM; i += kDThreads) out[(size_t)r * DIM + i] = NAN;
      if (weights_out)
        for (size_t i = tid; i < wrow; i += kDThreads) weights_out[(size_t)r * wrow + i] = 0.0f;
    }
    return;
  }
  const double *pmr = ws.pmax + rb;
  const uint32_t *ipr = ws.iphys + rb;
  double *xrow = ws.xs + (size_t)rb * P;
  uint32_t *xir = ws.xi + (size_t)rb * P;

  // 1. row maximum from the page maxima; a NaN maximum marks a malformed item
  double mx = -INFINITY;
  int nan = 0;
#pragma unroll 1
  for (int base = 0; base < cnt; base += 8 * kDThreads) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = pmr[min(base + u * kDThreads + tid, cnt - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) { mx = fmax(mx, v[u]); nan |= v[u] != v[u]; }
  }
  mx = block_max(mx, dred);
  nan = __syncthreads_or(nan);
  if (bad || nan) {
    if (c == 0) {
      if (tid == 0 && tau_out) tau_out[r] = NAN;
      for (int i = tid; i < DIM; i += kDThreads) out[(size_t)r * DIM + i] = NAN;
    }
    return;
  }
  const double thr = mx - 1.0;  // tau >= thr: F(mx - 1) >= 1

  EKV_MARK(1, 1);
  // 2. this chunk's candidates.  Pass 1 counts the chunk's scores above
  //    mx - 2^-i (i < 8); C tokens above mx - d give F(mx - d - C^-(alpha-1))
  //    >= C * (C^-(alpha-1))^(1/(alpha-1)) = 1, so each count certifies a
  //    lower bound on tau, valid for the whole row.  A lone block also keeps
  //    its candidates X > mx - 1 in LDS.  Each thread takes 8 consecutive
  //    tokens of one page (P is a multiple of 8), so one block scan per 2048
  //    tokens keeps the index order.
  const int tlo = (int)((long long)c * cnt / nsplit) * P, thi = (int)((long long)(c + 1) * cnt / nsplit) * P;
  const bool alone = nsplit == 1;
  double th[kNThr];
#pragma unroll
  for (int i = 0; i < kNThr; ++i) th[i] = mx - ldexp(1.0, -i);
  int cnt8[kNThr];
#pragma unroll
  for (int i = 0; i < kNThr; ++i) cnt8[i] = 0;
  int nlds = 0;
  // thread tid takes tokens base + 8 tid .. + 7 of each 2048-token step; the
  // first kKeepIt steps stay in registers for pass 2 (a chunk of up to 6144
  // tokens -- every chunk until a row keeps more than kSplitMax of them -- is
  // read once)
  double keep[kKeepIt][8];
  uint32_t keep_ph[kKeepIt];
  auto load8 = [&](int base, double (&v)[8], uint32_t &ph) __attribute__((always_inline)) {
    const int tc = min(base + 8 * tid, thi - 8);
    const double2 *src = reinterpret_cast<const double2 *>(xrow + tc);
#pragma unroll
    for (int h = 0; h < 4; ++h) { const double2 d2 = src[h]; v[2 * h] = d2.x; v[2 * h + 1] = d2.y; }
    ph = ipr[tc / P];
  };
  auto count8 = [&](int base, const double (&v)[8], uint32_t ph) __attribute__((always_inline)) {
    const int t0 = base + 8 * tid;
    const bool valid = t0 < thi;  // all 8 tokens or none (thi - t0 is a multiple of 8)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
#pragma unroll
      for (int i = 0; i < kNThr; ++i) cnt8[i] += (valid && v[u] > th[i]) ? 1 : 0;
    }
    if (alone) {
      int take = 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) take += (valid && v[u] > thr) ? 1 : 0;
      int tot;
      int at = nlds + block_excl_scan(take, scan_scratch, &tot);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (valid && v[u] > thr) {
          if (at < kCand) {
            const int t = t0 + u;
            cx[at] = v[u];
            ci[at] = t;
            cv[at] = (ph * (uint32_t)D.Hkv + (uint32_t)g) * (uint32_t)P + (uint32_t)(t % P);
          }
          ++at;
        }
      }
      nlds += tot;
    }
  };
#pragma unroll
  for (int it = 0; it < kKeepIt; ++it) {
    const int base = tlo + it * 8 * kDThreads;
    if (base < thi) {  // uniform
      load8(base, keep[it], keep_ph[it]);
      count8(base, keep[it], keep_ph[it]);
    }
  }
#pragma unroll 1
  for (int base = tlo + kKeepIt * 8 * kDThreads; base < thi; base += 8 * kDThreads) {
    double v[8];
    uint32_t ph;
    load8(base, v, ph);
    count8(base, v, ph);
  }
  // block totals of the counts, then the tightest certified bound
#pragma unroll
  for (int i = 0; i < kNThr; ++i) cnt8[i] = wave_sum(cnt8[i]);
  __syncthreads();
  if ((tid & (kWave - 1)) == 0)
    for (int i = 0; i < kNThr; ++i) s_cnt[tid / kWave][i] = cnt8[i];
  __syncthreads();
  // lane i (mod kNThr) evaluates threshold i's bound and a wave max combines
  // them: one reciprocal power per lane instead of kNThr in sequence (a chain
  // of dependent fp64 operations that dominates this phase otherwise)
  double Lc;
  {
    static_assert((kNThr & (kNThr - 1)) == 0, "kNThr is a power of two");
    const int i = tid & (kNThr - 1);
    int ci_ = 0;
    for (int w = 0; w < kDThreads / kWave; ++w) ci_ += s_cnt[w][i];
    const double cand =
        ci_ > 0 ? (mx - ldexp(1.0, -i)) - pow_neg_a((double)ci_, dp) - 1e-12 * fmax(1.0, fabs(mx)) : -INFINITY;
    Lc = fmax(thr, wave_max(cand));
  }
  if (!alone && tid < kNThr) {  // the chunk's counts, summed over the row by the last block
    int ct = 0;
    for (int w = 0; w < kDThreads / kWave; ++w) ct += s_cnt[w][tid];
    st_agent(&ws.segn[((size_t)r * kSplitMax + c) * kNThr + tid], ct);
  }
  const bool lds_all = alone && nlds <= kCand;  // every candidate X > mx - 1 is in LDS
  int total = nlds;                              // entries in the workspace segments (tiers 1, 2)
  double L = Lc;
  if (!lds_all) {
    // pass 2: compact X > Lc in place to the chunk's start (and into LDS when
    // alone); writes trail the reads, so no unread score is overwritten
    nlds = 0;
    int ncand = 0;
    auto compact8 = [&](int base, const double (&v)[8], uint32_t ph) __attribute__((always_inline)) {
      const int t0 = base + 8 * tid;
      const bool valid = t0 < thi;
      int take = 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) take += (valid && v[u] > Lc) ? 1 : 0;
      int tot;
      int at = ncand + block_excl_scan(take, scan_scratch, &tot);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (valid && v[u] > Lc) {
          const int t = t0 + u;
          st_agent(&xrow[tlo + at], v[u]);
          st_agent(&xir[tlo + at], (uint32_t)t);
          if (alone && at < kCand) {
            cx[at] = v[u];
            ci[at] = t;
            cv[at] = (ph * (uint32_t)D.Hkv + (uint32_t)g) * (uint32_t)P + (uint32_t)(t % P);
          }
          ++at;
        }
      }
      ncand += tot;
    };
#pragma unroll
    for (int it = 0; it < kKeepIt; ++it) {
      const int base = tlo + it * 8 * kDThreads;
      if (base < thi) compact8(base, keep[it], keep_ph[it]);
    }
#pragma unroll 1
    for (int base = tlo + kKeepIt * 8 * kDThreads; base < thi; base += 8 * kDThreads) {
      double v[8];
      uint32_t ph;
      load8(base, v, ph);
      compact8(base, v, ph);
    }
    total = ncand;
    nlds = alone ? ncand : 0;
  }
  EKV_MARK(1, 2);
  if (!alone) {
    if (tid == 0) {
      st_agent(&ws.segcnt[(size_t)r * kSplitMax + c], total);
      st_agent(&ws.segL[(size_t)r * kSplitMax + c], Lc);
    }
    if (!arrive_last(&ws.ctr[r], (unsigned)nsplit, &s_last)) return;
    EKV_MARK(1, 3);
    // the row's last block: segment offsets, the row's bound, then the
    // candidates above it into LDS
    // every chunk's hand-off is requested at once (one round trip): thread t
    // < nsplit kNThr takes count (chunk t / kNThr, threshold t % kNThr),
    // threads below nsplit also their chunk's candidate count and bound
    static_assert(kSplitMax * kNThr <= kDThreads, "one count per thread");
    const bool has_n = tid < nsplit * kNThr;
    int n_t = 0, c_t = 0;
    double l_t = 0.0;
    if (has_n) n_t = ld_agent(&ws.segn[((size_t)r * kSplitMax + tid / kNThr) * kNThr + tid % kNThr]);
    if (tid < nsplit) {
      c_t = ld_agent(&ws.segcnt[(size_t)r * kSplitMax + tid]);
      l_t = ld_agent(&ws.segL[(size_t)r * kSplitMax + tid]);
    }
    const bool ipr_lds = cnt <= kIprLds;  // the merge below looks pages up in LDS
    if (ipr_lds)
      for (int k = tid; k < cnt; k += kDThreads) s_ipr[k] = ipr[k];
    if (tid < kNThr) s_cnt[0][tid] = 0;
    __syncthreads();
    // the row's counts above mx - 2^-i are the chunks' counts summed (integer
    // adds, in any order): a bound as certified as each chunk's and tighter
    // (about sqrt(chunks) for alpha 1.5)
    if (has_n) atomicAdd(&s_cnt[0][tid % kNThr], n_t);
    // segment offsets (the first step's entry addresses need them): an
    // inclusive scan of the chunks' candidate counts across wave 0's lanes
    static_assert(kSplitMax <= kWave, "one chunk per lane of wave 0");
    if (tid < kWave) {
      int incl = tid < nsplit ? c_t : 0;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_up(incl, o, kWave);
        if (tid >= o) incl += v;
      }
      if (tid < nsplit) {
        soff[tid + 1] = incl;
        sL[tid] = l_t;
        sbase[tid] = (int)((long long)tid * cnt / nsplit) * P;
      }
      if (tid == 0) soff[0] = 0;
    }
    __syncthreads();
    total = soff[nsplit];
    const GlobSeg<1> gs0{xrow, soff, sbase, nsplit, total};
    // each thread takes 8 consecutive entries, so one block scan per 2048
    // entries keeps the candidates in index order; each step's scores and
    // token ids are requested one step ahead, so their round trip overlaps the
    // previous step's scan (the first step's, the row bound below)
    nlds = 0;
    auto ld8 = [&](int base, double (&v)[8], uint32_t (&t)[8]) __attribute__((always_inline)) {
      int a[8];
      gs0.addr_run<8>(base + 8 * tid, a);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        v[u] = ld_agent(&xrow[a[u]]);
        t[u] = ld_agent(&xir[a[u]]);
      }
    };
    double vn[8];
    uint32_t tn[8];
    if (total > 0) ld8(0, vn, tn);
    if (tid < kWave) {  // lane i (mod kNThr): threshold i's bound from the summed count
      const int i = tid & (kNThr - 1);
      const int ct = s_cnt[0][i];
      const double cand =
          ct > 0 ? (mx - ldexp(1.0, -i)) - pow_neg_a((double)ct, dp) - 1e-12 * fmax(1.0, fabs(mx)) : -INFINITY;
      const double cmax = wave_max(cand);
      if (tid == 0) {
        double lm = fmax(thr, cmax);
        for (int s2 = 0; s2 < nsplit; ++s2) lm = fmax(lm, sL[s2]);
        s_tau[0] = lm;
      }
    }
    lds_barrier();  // s_tau; the first step's loads stay in flight
    L = s_tau[0];
#pragma unroll 1
    for (int base = 0; base < total; base += 8 * kDThreads) {
      const int k0 = base + 8 * tid;
      double v[8];
      uint32_t t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) { v[u] = vn[u]; t[u] = tn[u]; }
      if (base + 8 * kDThreads < total) ld8(base + 8 * kDThreads, vn, tn);
      uint32_t ph[8];
      if (ipr_lds) {
#pragma unroll
        for (int u = 0; u < 8; ++u) ph[u] = s_ipr[min(t[u] / P, (uint32_t)(cnt - 1))];
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) ph[u] = ipr[t[u] / P];
      }
      int mine = 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) mine += (k0 + u < total && v[u] > L) ? 1 : 0;
      int tot;
      int at = nlds + block_excl_scan<true>(mine, scan_scratch, &tot);  // the next step's loads stay in flight
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (k0 + u < total && v[u] > L) {
          if (at < kCand) {
            cx[at] = v[u];
            ci[at] = (int)t[u];
            cv[at] = (ph[u] * (uint32_t)D.Hkv + (uint32_t)g) * (uint32_t)P + t[u] % P;
          }
          ++at;
        }
      }
      nlds += tot;
      if (nlds > kCand) break;  // the LDS set is only used when it holds them all (uniform)
    }
  } else if (tid == 0) {
    soff[0] = 0;
    soff[1] = total;
    sbase[0] = 0;
  }
  __syncthreads();
  EKV_MARK(1, 4);
  // candidate tiers: LDS (one wave solves), registers (block), workspace passes
  const int tier = nlds <= kCand ? 0 : ((total <= kRegPer * kDThreads && dp.ibeta != 0) ? 1 : 2);
  const int nsol = tier == 0 ? nlds : total;  // values the solver sees
  const int nseg = alone ? 1 : nsplit;
  const GlobSeg<1> gs{xrow, soff, sbase, nseg, total};
  double rx[kRegPer];
  uint32_t ri[kRegPer];
  if (tier == 1) {
#pragma unroll
    for (int j = 0; j < kRegPer; ++j) {
      const int a = gs.addr(min(tid * kRegPer + j, total - 1));
      rx[j] = ld_agent(&xrow[a]);
      ri[j] = ld_agent(&xir[a]);
    }
  }

  EKV_MARK(1, 5);
  // 3. threshold and normalizer
  double tau, z;
  if (dp.ibeta == 2) solve_row<2>(tier, dp, mx, L, nsol, cx, sortbuf, rx, gs, dred, &s_kstar, s_tau, tau, z);
  else if (dp.ibeta == 1) solve_row<1>(tier, dp, mx, L, nsol, cx, sortbuf, rx, gs, dred, &s_kstar, s_tau, tau, z);
  else solve_row<0>(tier, dp, mx, L, nsol, cx, sortbuf, rx, gs, dred, &s_kstar, s_tau, tau, z);
  EKV_MARK(1, 6);
  if (tid == 0 && tau_out) tau_out[r] = tau / dp.a;

  // 4. support gather, chunk by chunk in index order: compact (token, weight;
  //    V row when known), then kEpp entries at a time, kTpe threads per
  //    entry, each thread 8 coordinates with one 16-byte load; fixed-order
  //    final sum.
  const int ge = tid / kTpe, gc = tid % kTpe;
  float acc8[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc8[u] = 0.0f;
  int nsup = 0;
  const bool resolve = tier != 0;  // V rows looked up per flush from the item's physical page
  auto flush = [&]() __attribute__((always_inline)) {
    __syncthreads();
    if (resolve) {
      for (int k = tid; k < nsup; k += kDThreads) {
        const uint32_t t = (uint32_t)sup_i[k];
        sup_v[k] = (ipr[t / P] * (uint32_t)D.Hkv + (uint32_t)g) * (uint32_t)P + t % P;
      }
      __syncthreads();
    }
    int e = ge;
    // four entries per thread in flight, then two, then one
#pragma unroll 1
    for (; e + 3 * kEpp < nsup; e += 4 * kEpp) {
      float v0[8], v1[8], v2[8], v3[8];
      load_vec<8>(v_pool + (size_t)sup_v[e] * DIM + gc * 8, v0);
      load_vec<8>(v_pool + (size_t)sup_v[e + kEpp] * DIM + gc * 8, v1);
      load_vec<8>(v_pool + (size_t)sup_v[e + 2 * kEpp] * DIM + gc * 8, v2);
      load_vec<8>(v_pool + (size_t)sup_v[e + 3 * kEpp] * DIM + gc * 8, v3);
      const float w0 = sup_w[e], w1 = sup_w[e + kEpp], w2 = sup_w[e + 2 * kEpp], w3 = sup_w[e + 3 * kEpp];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc8[u] += w0 * v0[u];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc8[u] += w1 * v1[u];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc8[u] += w2 * v2[u];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc8[u] += w3 * v3[u];
    }
    if (e + kEpp < nsup) {
      float v0[8], v1[8];
      load_vec<8>(v_pool + (size_t)sup_v[e] * DIM + gc * 8, v0);
      load_vec<8>(v_pool + (size_t)sup_v[e + kEpp] * DIM + gc * 8, v1);
      const float w0 = sup_w[e], w1 = sup_w[e + kEpp];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc8[u] += w0 * v0[u];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc8[u] += w1 * v1[u];
      e += 2 * kEpp;
    }
    if (e < nsup) {
      float v0[8];
      load_vec<8>(v_pool + (size_t)sup_v[e] * DIM + gc * 8, v0);
      const float w0 = sup_w[e];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc8[u] += w0 * v0[u];
    }
    if (weights_out) {
      for (int k = tid; k < nsup; k += kDThreads) {
        const int pg = sel_idx[(size_t)r * MP + sup_i[k] / P];
        weights_out[(size_t)r * wrow + (size_t)pg * P + sup_i[k] % P] = sup_w[k];
      }
    }
    __syncthreads();
    nsup = 0;
  };
  // one compaction step over 256 entries (x, token, V row) in index order
  auto step = [&](double xk, int ik, uint32_t vk) __attribute__((always_inline)) {
    const double y = xk - tau;
    const int take = y > 0.0 ? 1 : 0;
    int tot;
    const int pos = block_excl_scan(take, scan_scratch, &tot);
    if (nsup + tot > kSupChunk) flush();
    if (take) {
      sup_v[nsup + pos] = vk;
      sup_i[nsup + pos] = ik;
      sup_w[nsup + pos] = (float)(pw_rt(y, dp) / z);
    }
    nsup += tot;
  };
  if (tier == 0) {
#pragma unroll 1
    for (int k0 = 0; k0 < nsol; k0 += kDThreads) {
      const int k = k0 + tid;
      step(k < nsol ? cx[k] : -INFINITY, k < nsol ? ci[k] : 0, k < nsol ? cv[k] : 0u);
    }
  } else if (tier == 1) {
    // each thread's support entries are consecutive in index order: one scan
    // places them all when they fit one gather pass
    int mine = 0;
#pragma unroll
    for (int j = 0; j < kRegPer; ++j) mine += (tid * kRegPer + j < total && rx[j] - tau > 0.0) ? 1 : 0;
    int stot;
    int at = block_excl_scan(mine, scan_scratch, &stot);
    if (stot <= kSupChunk) {
#pragma unroll
      for (int j = 0; j < kRegPer; ++j) {
        const double y = rx[j] - tau;
        if (tid * kRegPer + j < total && y > 0.0) {
          sup_i[at] = (int)ri[j];
          sup_w[at] = (float)(pw_rt(y, dp) / z);
          ++at;
        }
      }
      nsup = stot;
    } else {
      // registers rotate down one slot per step, so every access has a fixed index
#pragma unroll 1
      for (int j = 0; j < kRegPer; ++j) {
        step(tid * kRegPer + j < total ? rx[0] : -INFINITY, (int)ri[0], 0u);
#pragma unroll
        for (int u = 0; u + 1 < kRegPer; ++u) { rx[u] = rx[u + 1]; ri[u] = ri[u + 1]; }
      }
    }
  } else {
#pragma unroll 1
    for (int k0 = 0; k0 < total; k0 += kDThreads) {
      const int k = k0 + tid;
      const int a = gs.addr(min(k, total - 1));
      const double xv = ld_agent(&xrow[a]);
      const uint32_t t = ld_agent(&xir[a]);
      step(k < total ? xv : -INFINITY, (int)t, 0u);
    }
  }
  flush();
  EKV_MARK(1, 7);
#pragma unroll
  for (int u = 0; u < 8; ++u) accs[ge][gc * 8 + u] = acc8[u];
  __syncthreads();
  for (int cc = tid; cc < DIM; cc += kDThreads) {
    float s = accs[0][cc];
    for (int e = 1; e < kEpp; ++e) s += accs[e][cc];
    out[(size_t)r * DIM + cc] = s;
  }
}

static DecodeWs carve_decode(const Dims &D, long long cap, void *base, size_t *bytes) {
  Carve cv(base);
  const size_t rows = (size_t)D.B * D.Hq;
  DecodeWs w;
  w.xs = cv.take<double>((size_t)cap * D.P);
  w.xi = cv.take<uint32_t>((size_t)cap * D.P);
  w.pmax = cv.take<double>((size_t)cap);
  w.iphys = cv.take<uint32_t>((size_t)cap);
  w.rbase = cv.take<long long>(rows);
  w.segcnt = cv.take<int>(rows * kSplitMax);
  w.segL = cv.take<double>(rows * kSplitMax);
  w.segn = cv.take<int>(rows * kSplitMax * kNThr);
  w.ctr = cv.take<unsigned int>(rows);
  w.cap = cap;
  if (bytes) *bytes = cv.bytes();
  return w;
}

template <typename T, int DIM, int P>
static hipError_t launch_finish_t(const Dims &D, const DecodeParams &dp, const void *v_pool, const int32_t *seq_lens,
                                  const int32_t *sel_idx, const int32_t *sel_cnt, float *out, double *tau,
                                  float *weights_out, const DecodeWs &w, hipStream_t s) {
  const int rows = D.B * D.Hq;
  const size_t cand_bytes = (size_t)kCand * (8 + 4 + 4) + (dp.tau_method == 1 ? (size_t)kCand * 8 : 0);
  static bool attr_set = false;
  if (!attr_set) {
    const int most = (int)((size_t)kCand * (8 + 4 + 4 + 8));
    hipFuncSetAttribute((const void *)decode_finish_kernel<T, DIM, P, 2>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        most);
    hipFuncSetAttribute((const void *)decode_finish_kernel<T, DIM, P, 1>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        most);
    hipFuncSetAttribute((const void *)decode_finish_kernel<T, DIM, P, 0>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        most);
    attr_set = true;
  }
  const long long chunks = ((long long)D.max_pages * D.P + kChunkTok - 1) / kChunkTok;
  const int split = (int)(chunks < kSplitMax ? chunks : kSplitMax);
  const dim3 grid(rows, split);
  if (dp.ibeta == 2)
    hipLaunchKernelGGL((decode_finish_kernel<T, DIM, P, 2>), grid, dim3(kDThreads), cand_bytes, s, D, dp,
                       (const T *)v_pool, seq_lens, sel_idx, sel_cnt, out, tau, weights_out, w);
  else if (dp.ibeta == 1)
    hipLaunchKernelGGL((decode_finish_kernel<T, DIM, P, 1>), grid, dim3(kDThreads), cand_bytes, s, D, dp,
                       (const T *)v_pool, seq_lens, sel_idx, sel_cnt, out, tau, weights_out, w);
  else
    hipLaunchKernelGGL((decode_finish_kernel<T, DIM, P, 0>), grid, dim3(kDThreads), cand_bytes, s, D, dp,
                       (const T *)v_pool, seq_lens, sel_idx, sel_cnt, out, tau, weights_out, w);
  return hipGetLastError();
}

template <typename T, int DIM, int P>
static hipError_t launch_decode_t(const Dims &D, const DecodeParams &dp, const void *q,
                                  const void *k_pool, const void *v_pool, const int32_t *page_table,
                                  const int32_t *seq_lens, const int32_t *sel_idx,
                                  const int32_t *sel_cnt, float *out, double *tau,
                                  float *weights_out, void *ws, long long cap, hipStream_t s) {
  const DecodeWs w = carve_decode(D, cap, ws, nullptr);
  const int rows = D.B * D.Hq;
  const size_t map_bytes = (size_t)(rows + 1) * 4;
  hipLaunchKernelGGL((decode_scores_kernel<T, DIM, P>), dim3(kDGrid), dim3(kDThreads), map_bytes, s, D, dp,
                     (const T *)q, (const T *)k_pool, page_table, seq_lens, sel_idx, sel_cnt, weights_out, w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_finish_t<T, DIM, P>(D, dp, v_pool, seq_lens, sel_idx, sel_cnt, out, tau, weights_out, w, s);
}

template <typename T, int DIM>
static hipError_t launch_decode_p(const Dims &D, const DecodeParams &dp, const void *q, const void *k_pool,
                                  const void *v_pool, const int32_t *pt, const int32_t *sl, const int32_t *si,
                                  const int32_t *sc, float *out, double *tau, float *wo, void *ws, long long cap,
                                  hipStream_t s) {
  if (D.P == 16) return launch_decode_t<T, DIM, 16>(D, dp, q, k_pool, v_pool, pt, sl, si, sc, out, tau, wo, ws, cap, s);
  if (D.P == 32) return launch_decode_t<T, DIM, 32>(D, dp, q, k_pool, v_pool, pt, sl, si, sc, out, tau, wo, ws, cap, s);
  return launch_decode_t<T, DIM, 64>(D, dp, q, k_pool, v_pool, pt, sl, si, sc, out, tau, wo, ws, cap, s);
}

}  // namespace items

// the per-item decode into a workspace holding `cap` items (its bytes: decode_items_ws_bytes)
size_t decode_items_ws_bytes(const Dims &D, long long cap) {
  size_t b = 0;
  items::carve_decode(D, cap, nullptr, &b);
  return b;
}

hipError_t launch_entmax_decode_items(const Dims &D, int dtype, const void *q, const void *k_pool,
                                      const void *v_pool, const int32_t *page_table, const int32_t *seq_lens,
                                      const int32_t *sel_idx, const int32_t *sel_cnt, double alpha, int tau_method,
                                      float *out, double *tau, float *weights_out, void *ws, long long cap,
                                      hipStream_t s) {
  using namespace items;
  DecodeParams dp;
  dp.a = alpha - 1.0;
  dp.beta = 1.0 / dp.a;
  dp.c = D.scale;
  dp.ibeta = alpha == 1.5 ? 2 : (alpha == 2.0 ? 1 : 0);
  dp.tau_method = tau_method;
  if (dtype == ENTMAXKV_BF16) {
    if (D.d == 64)
      return launch_decode_p<uint16_t, 64>(D, dp, q, k_pool, v_pool, page_table, seq_lens, sel_idx, sel_cnt, out,
                                           tau, weights_out, ws, cap, s);
    return launch_decode_p<uint16_t, 128>(D, dp, q, k_pool, v_pool, page_table, seq_lens, sel_idx, sel_cnt, out, tau,
                                          weights_out, ws, cap, s);
  }
  if (D.d == 64)
    return launch_decode_p<float, 64>(D, dp, q, k_pool, v_pool, page_table, seq_lens, sel_idx, sel_cnt, out, tau,
                                      weights_out, ws, cap, s);
  return launch_decode_p<float, 128>(D, dp, q, k_pool, v_pool, page_table, seq_lens, sel_idx, sel_cnt, out, tau,
                                     weights_out, ws, cap, s);
}

EKV_TRACE_DUMP(ekv_trace_dump_decode_items)
}  // namespace ekv
