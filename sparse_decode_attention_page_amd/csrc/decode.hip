// decode.hip -- alpha-entmax attention over selected pages ([EntmaxKV s.2.C]).
//
// EntmaxKV s.2.C = section 2.C ("sparse entmax attention") of "Resumen Tecnico:
// EntmaxKV - Decodificacion Consciente del Soporte para Atencion Entmax",
// gist.science/es/paper/2605.21649: load only the KV entries of the selected
// pages and compute the alpha-entmax weights over that reduced set; when the
// selection contains the whole support the result is exact.
//
// alpha-entmax (Peters, Niculae & Martins 2019): with X_t = (alpha-1) s_t,
// p_t = [X_t - tau]_+^(1/(alpha-1)), tau the root of F(tau) = sum_t p_t = 1.
//
// The decode for many query-head rows, for sets per KV head and for the full
// cache (a set per query head over a few rows goes to decode_items.hip).  Two
// launches.
//  1. scores_kernel.  A block takes one KV head (b, g) and one slice of the
//     sequence's pages.  It finds each query head's kept pages inside the slice
//     (a 64-way search of the ascending set), merges them into the group's
//     union, reads each union page's K slice once and scores it for every head
//     of the group that kept it (bf16 products are exact in fp64; fp64 sums).
//     Scores pass through an LDS stage in batches; after each batch a head's
//     entries above (running max) - 1 are appended to its entries with their
//     V row.  F(max X - 1) >= 1, so tau >= max X - 1: no other token of the
//     row can carry weight, and the running max never exceeds the row's.
//     Per (row, slice) a summary: entry count, max, min, first position.
//  2. rows_kernel.  Up to nh blocks per row read the summaries and keep the
//     slices whose max exceeds the row's max - 1.  A row of at most 4096
//     entries is finished by one block from registers: a certified lower bound
//     on tau from counts above max - 2^-i, the candidates above it into LDS,
//     tau by Newton from the left with an exact last piece (or the sparsemax
//     sort form), then the V rows of the support; up to 16384 entries one
//     block takes them in rounds, each round tightening the bound.  Larger rows
//     are split into chunks that compact their candidates in place for the
//     row's last block, or, above 32768 entries, go through three steps, each
//     started by the previous one: an integer histogram of the entries, from
//     which bounds of F at the bin edges certify a window [e_lo, e_hi] holding
//     tau; the moments of the entries above e_hi and the entries inside the
//     window (the step's last block solves for tau exactly); the weighted V
//     gather, merged in chunk order.  A chunk waits only for its own row's last
//     block, every wait ends after a time limit (the row then reads NaN), and
//     every sum has a fixed order, so results repeat bit for bit.
//
// Full cache (the decode that reads every cached token, one of the baselines of
// the summary's efficiency results, section 4): the same two launches with the
// selection "every page", so K is read once per KV head and V for the support
// only.
#include <math.h>

#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace ekv {

constexpr int kDThreads = 256;
constexpr int kMaxSlices = 1024;  // slices per (b, g) at most
constexpr int kMaxR = 512;        // pages per slice at most (the page map of scores_kernel)
constexpr int kCand = 1024;       // candidates in LDS for the one-wave solve and the sort form
constexpr int kNThr = 8;          // count thresholds mx - 2^-i behind the certified bound on tau
constexpr int kHelpers = 32;      // helper blocks per row and step, at most
constexpr int kBins = 4096;       // histogram bins of a large row
constexpr int kSlot = 128;        // window entries a helper hands over
constexpr int kWin = 4096;        // window entries the solving helper keeps in LDS
constexpr unsigned kStMom = 3, kStGath = 4, kStDone = 0xFFu;  // steps of a large row (0: scores written)
constexpr unsigned long long kSpinTicks = 20000000ull;                     // 0.2 s of the 100 MHz clock
constexpr int kLargeN = 32768;  // rows with more entries take the histogram route
constexpr int kStStride = 32;  // row step flags 128 bytes apart, so waiting blocks of different rows poll different lines

struct DecodeWs {
  double *cx;         // [cap_tok]  entry X
  uint32_t *ct;       // [cap_tok]  the entry's V row: (physical page * Hkv + g) * P + slot
  uint32_t *cl;       // [cap_tok]  its logical position page * P + slot (written for weights_out only)
  int *s_cnt;         // [rows][ns] entries stored for the slice
  double *s_max;      // [rows][ns] max X over the slice's kept tokens (-inf: none; NaN: malformed)
  double *s_min;      // [rows][ns] min X over the slice's stored entries (+inf: none)
  uint32_t *s_start;  // [rows][ns] index in cx of the slice's first entry
  int *rcnt;          // [rows] items of the row (entries at most rcnt * P)
  unsigned *state;    // [rows][kStStride] step of a large row (one 128-byte line per row)
  unsigned *ctr;      // [rows][4] arrival counters of the helper steps and of the chunks
  double *rpar;       // [rows][8] published parameters (mx, lo, w, e_lo, e_hi, tau, z)
  double *crec;       // [rows][kHelpers][16] chunk records (entries kept, bound, counts, start, compacted)
  unsigned *hist;     // [rows][kBins]
  double *hpart;      // [rows][kHelpers][8] moment partials
  double *wbuf;       // [rows][kHelpers][kSlot] window entries handed over by each chunk
  float *opart;       // [rows][kHelpers][d] partial outputs
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

__device__ __forceinline__ double wave_min_d(double v) { return -wave_max(-v); }
__device__ __forceinline__ double block_min_d(double v, double *scratch) { return -block_max(-v, scratch); }

// Exclusive prefix sum over a block of a 64-bit value (fixed order).
template <bool kLdsOnly = false>
__device__ __forceinline__ unsigned long long block_excl_scan64(unsigned long long v, unsigned long long *scratch,
                                                                unsigned long long *total) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  unsigned long long x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const unsigned long long y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  block_sync<kLdsOnly>();
  if (lane == kWave - 1) scratch[w] = x;
  block_sync<kLdsOnly>();
  unsigned long long base = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    if (i < w) base += scratch[i];
    tot += scratch[i];
  }
  *total = tot;
  return base + x - v;
}

// Lower bounds of two keys in an ascending int list of n entries, by one wave:
// each round probes 64 evenly spaced entries and keeps the gap between the
// last probe below the key and the next one (one memory round trip per round;
// n <= 64 takes one round, n <= 4096 two).  A list that is not ascending gives
// some index in [0, n]; the caller checks the order of what it reads.
__device__ __forceinline__ void wave_bounds(const int32_t *list, int n, int key1, int key2, int *out1, int *out2) {
  const int lane = threadIdx.x & (kWave - 1);
  int lo1 = 0, hi1 = n, lo2 = 0, hi2 = n;
  while (hi1 > lo1 || hi2 > lo2) {
    const int st1 = (hi1 - lo1 + kWave - 1) / kWave, st2 = (hi2 - lo2 + kWave - 1) / kWave;
    const int q1 = lo1 + lane * st1, q2 = lo2 + lane * st2;
    const bool a1 = hi1 > lo1 && q1 < hi1, a2 = hi2 > lo2 && q2 < hi2;
    const int v1 = a1 ? list[q1] : 0;
    const int v2 = a2 ? list[q2] : 0;
    const int c1 = __popcll(__ballot(a1 && v1 < key1));
    const int c2 = __popcll(__ballot(a2 && v2 < key2));
    if (hi1 > lo1) {
      if (c1 == 0) {
        hi1 = lo1;
      } else {
        const int nlo = lo1 + (c1 - 1) * st1 + 1;
        hi1 = min(lo1 + c1 * st1, hi1);
        lo1 = nlo;
      }
    }
    if (hi2 > lo2) {
      if (c2 == 0) {
        hi2 = lo2;
      } else {
        const int nlo = lo2 + (c2 - 1) * st2 + 1;
        hi2 = min(lo2 + c2 * st2, hi2);
        lo2 = nlo;
      }
    }
  }
  *out1 = lo1;
  *out2 = lo2;
}

// =========================================================== 1. scores kernel
constexpr int kXl = 2048;  // X values a scores block stages in LDS (a batch of union pages)

// C consecutive K coordinates of one token as loaded (bf16: C/2 words, fp32: C
// words), converted to fp64 where they are used
template <typename T, int C>
struct KVec;
template <int C>
struct KVec<uint16_t, C> {
  uint32_t w[C / 2];
  __device__ __forceinline__ void load(const uint16_t *p) {
    if constexpr (C % 8 == 0) {
#pragma unroll
      for (int c = 0; c < C / 8; ++c) {
        const uint4 u = reinterpret_cast<const uint4 *>(p)[c];
        w[4 * c + 0] = u.x; w[4 * c + 1] = u.y; w[4 * c + 2] = u.z; w[4 * c + 3] = u.w;
      }
    } else {
      static_assert(C == 4, "bf16 coordinates come in fours or eights");
      const uint2 u = *reinterpret_cast<const uint2 *>(p);
      w[0] = u.x; w[1] = u.y;
    }
  }
  __device__ __forceinline__ double at(int i) const {
    return (double)((i & 1) ? bf16hi(w[i / 2]) : bf16lo(w[i / 2]));
  }
};
template <int C>
struct KVec<float, C> {
  float w[C];
  __device__ __forceinline__ void load(const float *p) {
#pragma unroll
    for (int c = 0; c < C / 4; ++c) {
      const float4 u = reinterpret_cast<const float4 *>(p)[c];
      w[4 * c + 0] = u.x; w[4 * c + 1] = u.y; w[4 * c + 2] = u.z; w[4 * c + 3] = u.w;
    }
  }
  __device__ __forceinline__ double at(int i) const { return (double)w[i]; }
};

// Lane pairings inside the lanes of one token: level J pairs lane e with
// e ^ m_J, m_J = 1, 2, 7, 15, 16 for J = 0..4 (two quad permutes, the mirrors
// inside 8 and 16 lanes, a swizzle across rows).  Each m_J has J as its top
// bit, so the pairings of J = L-1 .. 0 taken in turn join all 2^L lanes.
constexpr int pair_mask(int j) { return j == 0 ? 1 : j == 1 ? 2 : j == 2 ? 7 : j == 3 ? 15 : 16; }
template <int kCtrl>
__device__ __forceinline__ double mov_dpp_f64(double v) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp((int)(unsigned)u, kCtrl, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp((int)(unsigned)(u >> 32), kCtrl, 0xF, 0xF, true);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}
template <int kJ>
__device__ __forceinline__ double pair_f64(double v) {
  if constexpr (kJ == 0) return mov_dpp_f64<0xB1>(v);        // quad_perm [1,0,3,2]
  else if constexpr (kJ == 1) return mov_dpp_f64<0x4E>(v);   // quad_perm [2,3,0,1]
  else if constexpr (kJ == 2) return mov_dpp_f64<0x141>(v);  // row_half_mirror
  else if constexpr (kJ == 3) return mov_dpp_f64<0x140>(v);  // row_mirror
  else return __shfl_xor(v, 16, kWave);
}

// The per-head partials of a token's 2^L lanes are summed in L levels (level
// l pairs by m_J, J = L-1-l).  In the first lg G levels a lane keeps the lower
// half of its slots and adds its partner's upper half (a reduce-scatter); in
// the rest partners add their one slot.  Lane e holds head f(e) ^ i in slot i,
// with f linear over GF(2) and chosen so that partners line up:
// f(e ^ m_J) = f(e) ^ (slots handed over at that level), i.e. column J of f is
// that count xor the columns of m_J's lower bits.  Lane e ends with the full
// sum of head f(e); partners' sums take the same operands, so lanes of one
// head agree bit for bit.
constexpr int head_map_col(int L, int lg_g, int j) {
  const int l = L - 1 - j;
  int x = l < lg_g ? (1 << lg_g) >> (l + 1) : 0;
  for (int b = 0; b < j; ++b)
    if ((pair_mask(j) >> b) & 1) x ^= head_map_col(L, lg_g, b);
  return x;
}
// The columns are constants of the template (folded here: the recursive helper
// called at run time would make the kernel a non-leaf function).
template <int L, int kLgG, int J = 0>
__device__ __forceinline__ int head_map(int e) {
  if constexpr (J == L) {
    return 0;
  } else {
    constexpr int col = head_map_col(L, kLgG, J);
    return (((e >> J) & 1) ? col : 0) ^ head_map<L, kLgG, J + 1>(e);
  }
}
template <int kJ, int kV, int G>
__device__ __forceinline__ double head_sum_levels(double (&acc)[G]) {
  if constexpr (kJ < 0) {
    return acc[0];
  } else if constexpr (kV > 1) {
    constexpr int kH = kV / 2;
#pragma unroll
    for (int i = 0; i < kH; ++i) acc[i] += pair_f64<kJ>(acc[i + kH]);
    return head_sum_levels<kJ - 1, kH, G>(acc);
  } else {
    acc[0] += pair_f64<kJ>(acc[0]);
    return head_sum_levels<kJ - 1, 1, G>(acc);
  }
}

// max over the kSg lanes of the thread's team inside its wave (kSg = 32: the
// wave's halves, 64: the wave); uniform over the team.  All 64 lanes active.
template <int kSg>
__device__ __forceinline__ double team_max_w(double v) {
  v = fmax(v, dpp_f64<kDppXor1>(v));
  v = fmax(v, dpp_f64<kDppXor2>(v));
  v = fmax(v, dpp_f64<kDppRor4>(v));
  v = fmax(v, dpp_f64<kDppRor8>(v));
  const double m0 = fmax(readlane_f64(v, 0), readlane_f64(v, 16));
  const double m1 = fmax(readlane_f64(v, 32), readlane_f64(v, 48));
  if constexpr (kSg == 64) return fmax(m0, m1);
  else return (threadIdx.x & 32) ? m1 : m0;
}

struct KsArgs {
  const void *q, *k_pool;
  const int32_t *page_table, *seq_lens, *sel_idx, *sel_cnt;
  float *weights_out;
  int mode;            // 0: a set per query head; 1: a set per KV head; 2: every page
  int ns;              // slices per (b, g)
  long long item_cap;  // items the workspace holds
};

// items of row r: its count when in [0, N_b], else 0
__device__ __forceinline__ int ks_row_items(const Dims &D, const KsArgs &a, int r) {
  const int b = r / D.Hq;
  const int np = n_pages_of(seq_len_clamped(a.seq_lens, b, D), D.P);
  if (a.mode == 2) return np;
  const int c = a.mode == 0 ? a.sel_cnt[r] : a.sel_cnt[(size_t)b * D.Hkv + (r % D.Hq) / D.G];
  return (c < 0 || c > np) ? 0 : c;
}

template <typename T, int DIM, int P, int G>
__global__ __launch_bounds__(kDThreads)
void scores_kernel(Dims D, DecodeParams dp, KsArgs a, DecodeWs ws) {
  // scoring: kL lanes per token, kC coordinates each, q of the lane's
  // coordinates for every head in registers (fp64)
  constexpr int kC = 32 / G < 16 ? 32 / G : 16;
  constexpr int kLpt = DIM / kC;
  constexpr int kL = kLpt == 2 ? 1 : kLpt == 4 ? 2 : kLpt == 8 ? 3 : kLpt == 16 ? 4 : 5;
  constexpr int kLgG = G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3;
  constexpr int kTpp = kDThreads / kLpt;  // tokens per pass
  constexpr int kLdsTok = kXl / G;        // tokens per head in the LDS stage (a batch)
  constexpr int kXs = kLdsTok + 8;        // a head's stage row (padded: the heads' rows start in other banks)
  constexpr int kPpb = kLdsTok / kTpp;    // passes per batch
  constexpr int kKw = kC * (int)sizeof(T) / 4;
  constexpr int kRing = 32 / kKw >= 4 ? 4 : 2;  // K buffers in turn (kRing - 1 passes ahead)
  static_assert((1 << kL) == kLpt && kLpt >= G && kLpt <= 32, "a token's lanes split its heads");
  static_assert(kPpb % kRing == 0 && kLdsTok % P == 0, "a batch is whole passes and whole pages");
  static_assert(P % (kWave / kLpt) == 0, "a wave's tokens lie in one page");
  // compaction: a team of kS threads per head, kSg of them in one wave
  constexpr int kS = kDThreads / G;
  constexpr int kSg = kS < kWave ? kS : kWave;
  constexpr int kWpt = kS / kSg;          // waves per team
  constexpr int kTw = kLdsTok / kWpt;     // stage tokens per team wave
  constexpr int kGr = kTw / kSg;          // groups of kSg consecutive tokens
  static_assert(kSg == 32 || kSg == 64, "a team fills a wave or its halves");
  __shared__ unsigned umask[kMaxR];
  __shared__ int ulist[kMaxR];
  __shared__ uint32_t urow[kMaxR];   // union page: V row of its slot 0, (physical page * Hkv + g) * P
  __shared__ uint32_t uinfo[kMaxR];  // union page: heads that kept it | tokens << 8
  __shared__ int ptab[kMaxR];  // the slice's page-table entries
  __shared__ int s_lo[G], s_hi[G];
  __shared__ long long s_base[G];
  __shared__ int s_items[G];
  __shared__ unsigned s_bad, s_nu;
  __shared__ double s_tm[G][kWpt];  // per team wave: max (then min)
  __shared__ int s_tc[G][kWpt];     // per team wave: entries of the batch
  __shared__ long long red64[kDThreads / kWave];
  __shared__ int scan_scratch[kDThreads / kWave];
  __shared__ double xl[G * kXs];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int ns = a.ns;
  const int gi = blockIdx.x / ns, s = blockIdx.x % ns;
  const int b = gi / D.Hkv, g = gi % D.Hkv;
  const int r0 = b * D.Hq + g * G;
  const int MP = D.max_pages;
  const int L = seq_len_clamped(a.seq_lens, b, D);
  const int np = n_pages_of(L, P);
  const int R = max(1, (np + ns - 1) / ns);
  const int p0 = s * R;
  const T *q = (const T *)a.q;
  const T *k_pool = (const T *)a.k_pool;
  EKV_MARK(0, 0);
  // the slice's page-table entries, loaded beside the selection counts below
  int ptv[kMaxR / kDThreads];
#pragma unroll
  for (int i = 0; i < kMaxR / kDThreads; ++i) {
    const int o = tid + i * kDThreads;
    ptv[i] = (o < R && p0 + o < np) ? a.page_table[(size_t)b * MP + p0 + o] : -1;
  }
  // the lane's q coordinates, every head, slot i holding head hl ^ i
  const int e = tid % kLpt;
  const unsigned zt = (unsigned)(tid / kLpt);
  const int hl = head_map<kL, kLgG>(e);
  double qd[G][kC];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    float qf[kC];
    load_vec<kC>(q + (size_t)(r0 + (hl ^ i)) * DIM + e * kC, qf);
#pragma unroll
    for (int c = 0; c < kC; ++c) qd[i][c] = (double)qf[c];
  }

  // ---- the group's rows: first item (items of every earlier row), counts
  long long part = 0;
  for (int r = tid; r < r0; r += kDThreads) part += ks_row_items(D, a, r);
  part = block_sum(part, red64);
  if (tid == 0) {
    long long base = part;
    unsigned bad = 0;
    for (int h = 0; h < G; ++h) {
      const int r = r0 + h;
      const int raw = a.mode == 2 ? np : (a.mode == 0 ? a.sel_cnt[r] : a.sel_cnt[gi]);
      const int it = (raw < 0 || raw > np) ? 0 : raw;
      s_base[h] = base;
      s_items[h] = it;
      if (raw < 0 || raw > np || base + it > a.item_cap) bad |= 1u << h;
      base += it;
    }
    s_bad = (a.mode == 1 && bad) ? (1u << G) - 1u : bad;  // a group set serves all G rows
  }
  __syncthreads();

  // ---- each list's items inside the slice [p0, p0 + R) (the last slice takes the rest)
  const int nl = a.mode == 0 ? G : 1;
  const unsigned all = (1u << G) - 1u;
  if (a.mode == 2) {
    if (tid < G) {
      s_lo[tid] = min(p0, np);
      s_hi[tid] = min(p0 + R, np);
    }
  } else {
    for (int li = wv; li < nl; li += kDThreads / kWave) {
      const bool lbad = a.mode == 0 ? ((s_bad >> li) & 1u) != 0u : s_bad != 0u;
      const int n = lbad ? 0 : s_items[li];
      const int32_t *list = a.sel_idx + (size_t)(a.mode == 0 ? r0 + li : gi) * MP;
      int lo, hi;
      wave_bounds(list, n, p0, p0 + R, &lo, &hi);
      if (s == 0) lo = 0;
      if (s == ns - 1) hi = n;
      if (hi < lo) hi = lo;
      if (lane == 0) {
        s_lo[li] = lo;
        s_hi[li] = hi;
      }
    }
  }
  for (int o = tid; o < R; o += kDThreads) umask[o] = 0u;
#pragma unroll
  for (int i = 0; i < kMaxR / kDThreads; ++i) {
    const int o = tid + i * kDThreads;
    if (o < R) ptab[o] = ptv[i];
  }
  __syncthreads();
  if (a.mode == 2) {
    for (int o = tid; o < R; o += kDThreads)
      if (p0 + o < np) umask[o] = all;
  } else {
    for (int li = wv; li < nl; li += kDThreads / kWave) {
      const int32_t *list = a.sel_idx + (size_t)(a.mode == 0 ? r0 + li : gi) * MP;
      const int lo = s_lo[li], hi = s_hi[li];
      int bad = 0;
      for (int i = lo + lane; i < hi; i += kWave) {
        const int p = list[i];
        const int prev = i > 0 ? list[i - 1] : -1;
        const int o = p - p0;
        if (p < 0 || p >= np || p <= prev || o < 0 || o >= R) {
          bad = 1;
          continue;
        }
        atomicOr(&umask[o], a.mode == 0 ? (1u << li) : all);
      }
      if (__any(bad) && lane == 0) atomicOr(&s_bad, a.mode == 0 ? (1u << li) : all);
    }
  }
  __syncthreads();

  // ---- the union in page order (two offsets per thread) and its physical pages
  {
    const int o0 = 2 * tid;
    const int m0 = (o0 < R && umask[o0]) ? 1 : 0, m1 = (o0 + 1 < R && umask[o0 + 1]) ? 1 : 0;
    int tot;
    const int at = block_excl_scan(m0 + m1, scan_scratch, &tot);
    if (m0) ulist[at] = o0;
    if (m1) ulist[at + m0] = o0 + 1;
    if (tid == 0) s_nu = (unsigned)tot;
  }
  __syncthreads();
  const int nU = (int)s_nu;
  for (int k = tid; k < nU; k += kDThreads) {
    const int o = ulist[k];
    const int ph = ptab[o];
    const bool ok = ph >= 0 && ph < D.num_phys;
    urow[k] = ok ? ((uint32_t)ph * (uint32_t)D.Hkv + (uint32_t)g) * (uint32_t)P : 0u;
    uinfo[k] = umask[o] | (uint32_t)min(P, L - (p0 + o) * P) << 8;
    if (!ok) atomicOr(&s_bad, umask[o]);
  }
  __syncthreads();
  const unsigned live = all & ~s_bad;
  // weights_out: every slot of the slice's pages (the last slice to the end of
  // the row) is zeroed here; rows_kernel writes the support
  if (a.weights_out) {
    const size_t wrow = (size_t)MP * P;
    const size_t lo_s = (size_t)min(p0, MP) * P;
    const size_t hi_s = s == ns - 1 ? wrow : (size_t)min(p0 + R, MP) * P;
    for (int h = 0; h < G; ++h)
      for (size_t i = lo_s + tid; i < hi_s; i += kDThreads) a.weights_out[(size_t)(r0 + h) * wrow + i] = 0.0f;
  }
  // row bookkeeping of the rows_kernel (once per row)
  if (s == 0 && tid < G) {
    const int r = r0 + tid;
    ws.rcnt[r] = (s_bad >> tid) & 1u ? 0 : s_items[tid];
    ws.state[(size_t)r * kStStride] = 0u;
    ws.ctr[4 * r] = 0u;
    ws.ctr[4 * r + 1] = 0u;
    ws.ctr[4 * r + 2] = 0u;
    ws.ctr[4 * r + 3] = 0u;
  }
  // the histogram of a row that may take the histogram route starts at zero
  for (int h = 0; h < G; ++h)
    if (s == 0 && (long long)s_items[h] * P > kLargeN)
      for (int i = tid; i < kBins; i += kDThreads) ws.hist[(size_t)(r0 + h) * kBins + i] = 0u;
  EKV_MARK(0, 1);

  // ---- scores of the union pages' tokens, kTpp tokens per pass.  Union token
  // z (page z / P of the union, slot z % P) goes to the lane group zt of pass
  // z / kTpp; the lanes' per-head partials are summed by head_sum_levels, and
  // one lane per head and token puts its X into the LDS stage (-inf for heads
  // that did not keep the page and for slots past the sequence end; positions
  // past the union's last page are written but never read).
  const bool wr = (e & ((1 << (kL - kLgG)) - 1)) == 0;
  const int npass = (nU * P + kTpp - 1) / kTpp;
  const int nbatch = (npass + kPpb - 1) / kPpb;
  const unsigned ulast = (unsigned)max(nU - 1, 0);
  // every call issues its loads (past the last union page: that page again,
  // unused), so the count of loads in flight after a buffer's is fixed and its
  // wait leaves the later buffers' loads in flight
  auto load_pass = [&](int pass, KVec<T, kC> &kv) __attribute__((always_inline)) {
    const unsigned z = (unsigned)pass * kTpp + zt;
    const unsigned k = min(z / P, ulast);
    kv.load(k_pool + (size_t)(urow[k] + z % P) * DIM + e * kC);
  };
  auto score_pass = [&](int pass, const KVec<T, kC> &kv) __attribute__((always_inline)) {
    const unsigned z = (unsigned)pass * kTpp + zt;
    const unsigned k = z / P, t = z % P;
    const unsigned info = uinfo[min(k, ulast)];
    const unsigned m = k < (unsigned)nU ? (info & live) : 0u;
    double acc[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      acc[i] = kv.at(0) * qd[i][0];  // exact products
#pragma unroll
      for (int c = 1; c < kC; ++c) acc[i] = __builtin_fma(kv.at(c), qd[i][c], acc[i]);
    }
    const double sum = head_sum_levels<kL - 1, G, G>(acc);
    const double x = ((m >> hl) & 1u) && t < (info >> 8) ? dp.a * (dp.c * sum) : -INFINITY;
    if (wr) xl[hl * kXs + z % kLdsTok] = x;
  };

  // ---- a finished batch: head th's team reads the head's stage row, takes
  // its max into the running max and appends the entries above (running max)
  // - 1 to the head's entries, in index order (ballots inside each group of kSg
  // consecutive tokens; the team's waves take consecutive shares).  The running
  // max never exceeds the slice max, so the stored entries hold every entry
  // above (slice max) - 1.
  const int th = tid / kS, tw = (tid % kS) / kSg, tl = lane % kSg;
  const unsigned long long tmask = kSg == kWave ? ~0ull : (((1ull << kSg) - 1ull) << (lane & kSg));
  const unsigned long long below = (1ull << lane) - 1ull;
  const size_t hbase = (size_t)(s_base[th] + s_lo[a.mode == 0 ? th : 0]) * P;
  double rmax = -INFINITY, mn = INFINITY;
  int ncnt = 0;
  auto compact_batch = [&](int bt) __attribute__((always_inline)) {
    lds_barrier();  // the batch's stage writes before the reads below
    const int kb0 = bt * (kLdsTok / P);
    double v[kGr];
    double bm = -INFINITY;
#pragma unroll
    for (int i = 0; i < kGr; ++i) {
      const int zl = tw * kTw + i * kSg + tl;
      v[i] = kb0 + zl / P < nU ? xl[th * kXs + zl] : -INFINITY;
      bm = fmax(bm, v[i]);
    }
    bm = team_max_w<kSg>(bm);
    if constexpr (kWpt > 1) {
      if (tl == 0) s_tm[th][tw] = bm;
      lds_barrier();
#pragma unroll
      for (int w = 0; w < kWpt; ++w) bm = fmax(bm, s_tm[th][w]);
    }
    rmax = fmax(rmax, bm);
    const double thr = rmax - 1.0;
    int pre = 0, tot = 0;  // entries of the team's earlier waves, of the whole team
    if constexpr (kWpt > 1) {
      int cw = 0;
#pragma unroll
      for (int i = 0; i < kGr; ++i) cw += __popcll(__ballot(v[i] > thr) & tmask);
      if (tl == 0) s_tc[th][tw] = cw;
      lds_barrier();
#pragma unroll
      for (int w = 0; w < kWpt; ++w) {
        const int c = s_tc[th][w];
        pre += w < tw ? c : 0;
        tot += c;
      }
    }
    size_t at = hbase + ncnt + pre;
#pragma unroll
    for (int i = 0; i < kGr; ++i) {
      const bool keep = v[i] > thr;
      const unsigned long long bal = __ballot(keep) & tmask;
      if (keep) {
        const int zl = tw * kTw + i * kSg + tl;
        const int k = kb0 + zl / P, t = zl % P;
        const size_t w = at + __popcll(bal & below);
        ws.cx[w] = v[i];
        ws.ct[w] = urow[k] + (uint32_t)t;
        if (a.weights_out) ws.cl[w] = (uint32_t)((p0 + ulist[k]) * P + t);
        mn = fmin(mn, v[i]);
      }
      at += __popcll(bal);
    }
    ncnt += kWpt > 1 ? tot : (int)(at - hbase - ncnt);
    lds_barrier();  // the stage is read before the next batch overwrites it
  };

  // ---- the passes, kRing K buffers used in turn (no register copies, which
  // would wait for loads still in flight), kRing - 1 passes ahead
  KVec<T, kC> kb[kRing];
  if (npass > 0) {
#pragma unroll
    for (int i = 0; i < kRing - 1; ++i) load_pass(i, kb[i]);
    for (int bt = 0; bt < nbatch; ++bt) {
      const int pe = min(npass, (bt + 1) * kPpb);
#pragma unroll 1
      for (int p = bt * kPpb; p < pe; p += kRing) {
#pragma unroll
        for (int i = 0; i < kRing; ++i) {
          load_pass(p + i + kRing - 1, kb[(i + kRing - 1) % kRing]);
          score_pass(p + i, kb[i]);
        }
      }
      compact_batch(bt);
    }
  }
  // ---- per (row, slice) summary: entry count, max, min of the stored entries
  mn = -team_max_w<kSg>(-mn);
  if constexpr (kWpt > 1) {
    if (tl == 0) s_tm[th][tw] = mn;
    lds_barrier();
#pragma unroll
    for (int w = 0; w < kWpt; ++w) mn = fmin(mn, s_tm[th][w]);
  }
  if (tid % kS == 0) {
    const int h = th, r = r0 + h;
    const bool bad = (s_bad >> h) & 1u;
    const size_t o = (size_t)r * ns + s;
    ws.s_cnt[o] = bad ? 0 : ncnt;
    ws.s_max[o] = bad ? NAN : rmax;
    ws.s_min[o] = mn;
    ws.s_start[o] = bad ? 0u : (uint32_t)hbase;
  }
  EKV_MARK(0, 2);
}

// ================================================================ 2. rows kernel
struct RowsArgs {
  const void *v_pool;
  float *out;
  double *tau;
  float *weights_out;
  int ns, nh;  // slices per row; blocks (chunks at most) per row
};

// The entries of a run of slices, concatenated in index order, by a window
// [off, off + n] of an LDS table of entry offsets (ascending; off[0] may be
// nonzero) and first positions: entry k of the run is slice i's entry
// k + off[0] - off[i], at cx[start[i] + k + off[0] - off[i]] (its V row at ct,
// its position at cl, same index).
struct Segs {
  const int *off;         // [n + 1]
  const uint32_t *start;  // [n]
  int n, total, e0;
  __device__ __forceinline__ int seg_of(int k) const {
    int lo = 0, hi = n - 1;  // last slice starting at or before k
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] - e0 <= k) lo = mid; else hi = mid - 1;
    }
    return lo;
  }
  // addresses of entries min(k0 + u, total - 1), u < R (total > 0): one
  // search, then the slice advances with k (empty slices are stepped over)
  template <int R>
  __device__ __forceinline__ void addr_run(int k0, size_t (&ad)[R]) const {
    int lo = seg_of(min(k0, total - 1));
    int next = lo + 1 < n ? off[lo + 1] - e0 : 0x7fffffff;
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int k = min(k0 + u, total - 1);
      while (k >= next) {
        ++lo;
        next = lo + 1 < n ? off[lo + 1] - e0 : 0x7fffffff;
      }
      ad[u] = (size_t)start[lo] + (size_t)(k + e0 - off[lo]);
    }
  }
};
// entries k0 + u * kDThreads, u < R (those past the end: the last entry),
// each found by its own fixed-step search of the table, all R side by side
template <int R>
__device__ __forceinline__ void addr_strided(const Segs &sg, int k0, size_t (&ad)[R]) {
  int lo[R], kk[R];
#pragma unroll
  for (int u = 0; u < R; ++u) {
    lo[u] = 0;
    kk[u] = min(k0 + u * kDThreads, sg.total - 1) + sg.e0;
  }
  int step = 1;
  while (2 * step < sg.n) step <<= 1;
#pragma unroll 1
  for (; step > 0; step >>= 1) {
    int v[R];
#pragma unroll
    for (int u = 0; u < R; ++u) v[u] = sg.off[min(lo[u] + step, sg.n - 1)];  // every read issued first
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const bool go = (lo[u] + step < sg.n) & (v[u] <= kk[u]);  // no short circuit: the reads stay unconditional
      lo[u] += go ? step : 0;
    }
  }
#pragma unroll
  for (int u = 0; u < R; ++u) ad[u] = (size_t)sg.start[lo[u]] + (size_t)(kk[u] - sg.off[lo[u]]);
}

// the run of table entries [t0, t1) (the table visible to every thread)
__device__ __forceinline__ Segs segs_window(const int *off, const uint32_t *start, int t0, int t1) {
  Segs sg;
  sg.off = off + t0;
  sg.start = start + t0;
  sg.n = t1 - t0;
  sg.e0 = off[t0];
  sg.total = off[t1] - sg.e0;
  return sg;
}

// Eight consecutive entries per thread (X, and token ids when asked);
// entries past the end read -inf.
struct Batch8 {
  double v[8];
  uint32_t t[8];  // V rows
};
__device__ __forceinline__ void load_batch8(const Segs &sg, const DecodeWs &ws, int k0, bool toks, bool agent,
                                            Batch8 &bt) {
  if (k0 < sg.total) {
    size_t ad[8];
    sg.addr_run<8>(k0, ad);
#pragma unroll
    for (int u = 0; u < 8; ++u) bt.v[u] = agent ? ld_agent(&ws.cx[ad[u]]) : ws.cx[ad[u]];
    if (toks)
#pragma unroll
      for (int u = 0; u < 8; ++u) bt.t[u] = agent ? ld_agent(&ws.ct[ad[u]]) : ws.ct[ad[u]];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (k0 + u >= sg.total) bt.v[u] = -INFINITY;
  } else {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      bt.v[u] = -INFINITY;
      bt.t[u] = 0u;
    }
  }
}

// fn over every batch of sg's entries (eight per thread, 2048 per batch) in
// order, the next batch's loads issued before fn runs on the current one; two
// buffers used in turn (copying a buffer would wait for its loads).  fn may
// hold block barriers: every thread makes the same calls.
template <typename Fn>
__device__ __forceinline__ void stream_batches(const Segs &sg, const DecodeWs &ws, bool toks, bool agent, Fn &&fn) {
  constexpr int kStep = 8 * kDThreads;
  const int M = sg.total, t8 = 8 * (int)threadIdx.x;
  Batch8 b0, b1;
  load_batch8(sg, ws, t8, toks, agent, b0);
#pragma unroll 1
  for (int base = 0; base < M; base += 2 * kStep) {
    if (base + kStep < M) load_batch8(sg, ws, base + kStep + t8, toks, agent, b1);
    fn(b0);
    if (base + kStep >= M) break;
    if (base + 2 * kStep < M) load_batch8(sg, ws, base + 2 * kStep + t8, toks, agent, b0);
    fn(b1);
  }
}

// ------------------------------------------------------------- threshold solve
// Values seen by the solver: LDS entries (strided over the participating
// threads), registers, or every entry of a row in the workspace.
struct LdsVals {
  const double *v;
  int n, t0, stride;
  template <typename Fn>
  __device__ __forceinline__ void each(Fn &&fn) const {
#pragma unroll 2
    for (int i = t0; i < n; i += stride) fn(v[i]);
  }
};
struct RegVals16 {  // 16 values per thread (-inf for unused slots)
  const double (&v)[16];
  template <typename Fn>
  __device__ __forceinline__ void each(Fn &&fn) const {
#pragma unroll
    for (int j = 0; j < 16; ++j) fn(v[j]);
  }
};
struct GlobVals {  // every entry of a run of slices, 8 per thread in flight
  const DecodeWs *ws;
  const Segs *sg;
  bool agent;       // entries another block of the launch may have rewritten
  template <typename Fn>
  __device__ __forceinline__ void each(Fn &&fn) const {
#pragma unroll 1
    for (int base = 0; base < sg->total; base += 8 * kDThreads) {
      const int k0 = base + 8 * (int)threadIdx.x;
      if (k0 >= sg->total) continue;
      size_t ad[8];
      sg->addr_run<8>(k0, ad);
      double v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = agent ? ld_agent(&ws->cx[ad[u]]) : ws->cx[ad[u]];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (k0 + u < sg->total) fn(v[u]);
    }
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

// Entries known only through their moments: m0 entries above e with
// m1 = sum (x - e), m2 = sum (x - e)^2 and ymin = min (x - e) (m0 = 0: none).
struct Above {
  double m0, m1, m2, ymin, e;
};

// Root of F(t) = sum [X - t]_+^beta = 1 by Newton from the left: lo0 has
// F >= 1 (a certified lower bound), hi has F <= 1.  For alpha <= 2 (beta >= 1)
// F is convex and decreasing, so every Newton iterate from the left stays left
// of the root: one pass per step.  Otherwise each Newton candidate is checked
// with a second pass; one that leaves (lo, hi) becomes a bisection step, and
// after a step lands right of the root the next step bisects.
//
// alpha = 2 and 1.5 (beta = 1, 2): between consecutive scores F is linear or
// quadratic, F(lo + u) = sum_A (y - u)^beta over the active set A = {y = X - lo
// > 0}.  Each pass also solves that piece exactly (u = (S1 - 1)/|A|, or the
// smaller root (S2 - 1)/(S1 + sqrt(S1^2 - |A|(S2 - 1))) of |A| u^2 - 2 S1 u + S2
// = 1); when u <= min_A y every active score stays active at lo + u, so lo + u
// is F's root and the pass ends the search (*z_out = F there, from the same
// sums).  The entries of `ab` (all above hi, so active throughout) enter the
// sums through their moments.  *z_out = 0 when the search ends another way.
template <int kB, typename Src, typename Red>
__device__ __forceinline__ double newton_tau(const Src &src, const Above &ab, double lo0, double hi,
                                             const DecodeParams &dp, double *dred, double *z_out) {
  const Red red;
  double lo = lo0;
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
      if (ab.m0 > 0.0) {
        const double d = ab.e - lo;  // >= 0
        sm[0] += ab.m1 + d * ab.m0;
        sm[1] += ab.m2 + (2.0 * d) * ab.m1 + (d * d) * ab.m0;
        sm[2] += ab.m0;
        nmn = fmax(nmn, -(ab.ymin + d));
      }
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

// tau and z = F(tau) over a source by the whole block; ab as in newton_tau
// (m0 > 0 only for alpha = 1.5, 2).
template <typename Src>
__device__ __forceinline__ void solve_block(const Src &src, const Above &ab, double lo0, double hi, const DecodeParams &dp,
                            double *dred, double &tau, double &z) {
  double zk = 0.0;
  if (dp.ibeta == 2) tau = newton_tau<2, Src, BlockRed>(src, ab, lo0, hi, dp, dred, &zk);
  else if (dp.ibeta == 1) tau = newton_tau<1, Src, BlockRed>(src, ab, lo0, hi, dp, dred, &zk);
  else tau = newton_tau<0, Src, BlockRed>(src, ab, lo0, hi, dp, dred, &zk);
  if (zk > 0.0) {
    z = zk;
    return;
  }
  double zz = 0.0;
  src.each([&](double x) { const double y = x - tau; if (y > 0.0) zz += pw_rt(y, dp); });
  if (ab.m0 > 0.0 && threadIdx.x == 0) {  // the moment entries: sum (y + d)^beta in closed form
    const double d = ab.e - tau;
    zz += dp.ibeta == 2 ? ab.m2 + (2.0 * d) * ab.m1 + (d * d) * ab.m0 : ab.m1 + d * ab.m0;
  }
  z = block_sum(zz, dred);
}

// sparsemax closed form (Martins & Astudillo 2016) by a bitonic sort in LDS:
// sort z descending; k* = max{k : 1 + k z_(k) > sum_{j<=k} z_(j)};
// tau = (sum_{j<=k*} z_(j) - 1) / k*.  The condition holds exactly for k <= k*.
// Only the candidates are sorted: every score outside them is below tau.
__device__ __forceinline__ double sparsemax_tau_sort(const double *cx, int n, double *buf, double *dred, int *s_kstar) {
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

// ------------------------------------------------------------- support gather
// Support entries are placed in LDS by block scans (in the order they are
// offered); a flush accumulates p_t v_t over them: kEpp entries per pass with
// kTpe threads each (8 coordinates per 16-byte load), fp32 in a fixed order.
constexpr int kSupCap = 2048;  // support entries held in LDS between flushes
template <typename T, int DIM>
struct GatherLds {
  static constexpr int kTpe = DIM / 8;           // threads per support entry
  static constexpr int kEpp = kDThreads / kTpe;  // support entries per gather pass
  uint32_t vrow[kSupCap];
  float w[kSupCap];
  float accs[kEpp][DIM + 1];
};

template <typename T, int DIM>
struct Gather {
  static constexpr int kTpe = GatherLds<T, DIM>::kTpe;
  static constexpr int kEpp = GatherLds<T, DIM>::kEpp;
  GatherLds<T, DIM> *sh;
  int *scan_scratch;
  const T *v_pool;
  double tau, z;
  DecodeParams dp;
  int nsup;
  float acc8[8];

  __device__ __forceinline__ void flush() {
    lds_barrier();
    const int tid = threadIdx.x, ge = tid / kTpe, gc = tid % kTpe;
    int e = ge;
    // eight entries per thread in flight, then four, two, one (the sum runs
    // over e, e + kEpp, e + 2 kEpp, ... in that order either way)
#pragma unroll 1
    for (; e + 7 * kEpp < nsup; e += 8 * kEpp) {
      float v[8][8];
#pragma unroll
      for (int i = 0; i < 8; ++i) load_vec<8>(v_pool + (size_t)sh->vrow[e + i * kEpp] * DIM + gc * 8, v[i]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float wi = sh->w[e + i * kEpp];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc8[u] += wi * v[i][u];
      }
    }
    if (e + 3 * kEpp < nsup) {
      float v0[8], v1[8], v2[8], v3[8];
      load_vec<8>(v_pool + (size_t)sh->vrow[e] * DIM + gc * 8, v0);
      load_vec<8>(v_pool + (size_t)sh->vrow[e + kEpp] * DIM + gc * 8, v1);
      load_vec<8>(v_pool + (size_t)sh->vrow[e + 2 * kEpp] * DIM + gc * 8, v2);
      load_vec<8>(v_pool + (size_t)sh->vrow[e + 3 * kEpp] * DIM + gc * 8, v3);
      const float w0 = sh->w[e], w1 = sh->w[e + kEpp], w2 = sh->w[e + 2 * kEpp], w3 = sh->w[e + 3 * kEpp];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc8[u] += w0 * v0[u];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc8[u] += w1 * v1[u];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc8[u] += w2 * v2[u];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc8[u] += w3 * v3[u];
      e += 4 * kEpp;
    }
    if (e + kEpp < nsup) {
      float v0[8], v1[8];
      load_vec<8>(v_pool + (size_t)sh->vrow[e] * DIM + gc * 8, v0);
      load_vec<8>(v_pool + (size_t)sh->vrow[e + kEpp] * DIM + gc * 8, v1);
      const float w0 = sh->w[e], w1 = sh->w[e + kEpp];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc8[u] += w0 * v0[u];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc8[u] += w1 * v1[u];
      e += 2 * kEpp;
    }
    if (e < nsup) {
      float v0[8];
      load_vec<8>(v_pool + (size_t)sh->vrow[e] * DIM + gc * 8, v0);
      const float w0 = sh->w[e];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc8[u] += w0 * v0[u];
    }
    lds_barrier();
    nsup = 0;
  }
  // up to R entries of this thread (X, V row), consecutive in index order
  // (R * 256 <= kSupCap); one block scan places the block's support entries
  template <int R>
  __device__ __forceinline__ void offer(const double (&x)[R], const uint32_t (&vr)[R]) {
    static_assert(R * kDThreads <= kSupCap, "one offer fits the buffer");
    int take = 0;
#pragma unroll
    for (int u = 0; u < R; ++u) take += x[u] - tau > 0.0 ? 1 : 0;
    int tot;
    int at = block_excl_scan<true>(take, scan_scratch, &tot);  // loads issued before stay in flight
    if (nsup + tot > kSupCap) flush();                          // uniform
    at += nsup;
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const double y = x[u] - tau;
      if (y > 0.0) {
        sh->vrow[at] = vr[u];
        sh->w[at] = (float)(pw_rt(y, dp) / z);
        ++at;
      }
    }
    nsup += tot;
  }
  // the block's sum of p_t v_t into dst[0 .. DIM) (fixed order)
  __device__ __forceinline__ void finish(float *dst, bool agent) {
    flush();
    const int tid = threadIdx.x, ge = tid / kTpe, gc = tid % kTpe;
#pragma unroll
    for (int u = 0; u < 8; ++u) sh->accs[ge][gc * 8 + u] = acc8[u];
    __syncthreads();
    for (int cc = tid; cc < DIM; cc += kDThreads) {
      float s = sh->accs[0][cc];
      for (int e = 1; e < kEpp; ++e) s += sh->accs[e][cc];
      if (agent) st_agent(&dst[cc], s);
      else dst[cc] = s;
    }
  }
};

template <typename T, int DIM>
__device__ __forceinline__ Gather<T, DIM> make_gather(GatherLds<T, DIM> *sh, int *scan_scratch, const DecodeParams &dp,
                                                      const RowsArgs &ra, double tau, double z) {
  Gather<T, DIM> ga;
  ga.sh = sh;
  ga.scan_scratch = scan_scratch;
  ga.v_pool = (const T *)ra.v_pool;
  ga.tau = tau;
  ga.z = z;
  ga.dp = dp;
  ga.nsup = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) ga.acc8[u] = 0.0f;
  return ga;
}

// Support gather over the entries of sg (eight per thread per step, the next
// eight in flight); the block's partial output goes to dst.
template <typename T, int DIM>
__device__ __forceinline__ void gather_entries(Gather<T, DIM> &ga, const Segs &sg, const DecodeWs &ws, bool agent) {
  stream_batches(sg, ws, true, agent, [&](const Batch8 &bt) __attribute__((always_inline)) {
    ga.template offer<8>(bt.v, bt.t);
  });
}

// weights_out: p_t of every entry of sg above tau, at its position
__device__ __forceinline__ void write_weights(const Segs &sg, const DecodeWs &ws, float *wrow, double tau, double z,
                                              const DecodeParams &dp, bool agent) {
#pragma unroll 1
  for (int k = threadIdx.x; k < sg.total; k += kDThreads) {
    size_t ad[1];
    sg.addr_run<1>(k, ad);
    const double y = (agent ? ld_agent(&ws.cx[ad[0]]) : ws.cx[ad[0]]) - tau;
    if (y > 0.0) wrow[agent ? ld_agent(&ws.cl[ad[0]]) : ws.cl[ad[0]]] = (float)(pw_rt(y, dp) / z);
  }
}

// Waits until the row's step is at least `need` (kStDone counts); returns the
// step seen, or 0 after the time limit.
__device__ __forceinline__ unsigned wait_step(const unsigned *state, unsigned need, unsigned *s_flag) {
  if (threadIdx.x == 0) {
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    unsigned v;
    for (;;) {
      v = ld_agent(state);
      if (v >= need) break;
      if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinTicks) {
        v = 0u;
        break;
      }
      __builtin_amdgcn_s_sleep(8);  // about 0.2 us between polls
    }
    *s_flag = v;
  }
  __syncthreads();
  return *s_flag;
}

__device__ __forceinline__ void publish_step(unsigned *state, unsigned v) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) st_agent(state, v);
}

template <int DIM>
__device__ __forceinline__ void row_nan(const RowsArgs &ra, int r) {
  for (int i = threadIdx.x; i < DIM; i += kDThreads) ra.out[(size_t)r * DIM + i] = NAN;
  if (threadIdx.x == 0 && ra.tau) ra.tau[r] = NAN;
}

// an empty row: zero output, tau NaN
template <int DIM>
__device__ __forceinline__ void row_empty(const RowsArgs &ra, int r) {
  for (int i = threadIdx.x; i < DIM; i += kDThreads) ra.out[(size_t)r * DIM + i] = 0.0f;
  if (threadIdx.x == 0 && ra.tau) ra.tau[r] = NAN;
}

// LDS of the rows kernel (one layout per role, overlaid)
template <typename T, int DIM>
struct RowsLds {
  int off[kMaxSlices + 1];      // the row's non-empty slices: entry offsets (ascending), then N
  uint32_t start[kMaxSlices];   // and their first positions in cx
  int moff[kHelpers + 1];       // compacted chunk runs: entry offsets (a chunk left in place adds 0)
  uint32_t mst[kHelpers];       // and first positions
  union {
    struct {
      double cx[kCand];
      uint32_t cv[kCand];
      union {
        GatherLds<T, DIM> ga;
        double sortbuf[kCand];
      };
    } lead;
    unsigned hist[kBins];
    double win[kWin];
    GatherLds<T, DIM> ga;
  };
};

// ------------------------------------------------------------ chunk blocks
// Chunk c of nc holds the table entries t whose entries-before count off[t]
// maps to c (floor(off[t] nc / N)); [t0, t1) by two searches of the table.
__device__ __forceinline__ void chunk_window(const int *off, int ntab, int N, int nc, int c, int *t0, int *t1) {
  auto first_ge = [&](int cc) __attribute__((always_inline)) {
    int lo = 0, hi = ntab;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((long long)off[mid] * nc / N >= cc) hi = mid; else lo = mid + 1;
    }
    return lo;
  };
  *t0 = (c == 0 || N == 0) ? 0 : first_ge(c);
  *t1 = (c == nc - 1 || N == 0) ? ntab : first_ge(c + 1);
}

// After the chunk step: chunk c's entries, compacted (one run at mst[c], its
// entries read back through agent-scope loads) or in place (its window of the
// row's table).  s_rec holds the chunks' records.
__device__ __forceinline__ Segs chunk_segs(const int *off, const uint32_t *start, const int *moff,
                                           const uint32_t *mst, const double (*s_rec)[13], int ntab, int N, int nc,
                                           int c) {
  if (s_rec[c][11] != 0.0) return segs_window(moff, mst, c, c + 1);
  int t0, t1;
  chunk_window(off, ntab, N, nc, c, &t0, &t1);
  return segs_window(off, start, t0, t1);
}

// Every entry of row r, chunk by chunk (agent-scope loads: compacted runs
// were written by other blocks of the launch)
struct RowVals {
  const DecodeWs *ws;
  const int *off, *moff;
  const uint32_t *start, *mst;
  const double (*s_rec)[13];
  int ntab, N, nc;
  template <typename Fn>
  __device__ __forceinline__ void each(Fn &&fn) const {
#pragma unroll 1
    for (int c = 0; c < nc; ++c) {
      const Segs sg = chunk_segs(off, start, moff, mst, s_rec, ntab, N, nc, c);
      const GlobVals gv{ws, &sg, true};
      gv.each(fn);
    }
  }
};

// Row tau and z from every entry by passes over the workspace (generic
// exponent with many candidates, or a window too wide for the slots); with
// `gather` the support gather, the output and weights_out too.
template <typename T, int DIM>
__device__ __forceinline__ void row_slow(const DecodeParams &dp, const RowsArgs &ra, const DecodeWs &ws, int r,
                                         RowsLds<T, DIM> &sm, const RowVals &src, double lo0, double hi, double *dred,
                                         int *scan_scratch, float *wrow, bool gather, double *tau_o, double *z_o) {
  const Above none{0.0, 0.0, 0.0, 0.0, 0.0};
  double tau, z;
  solve_block(src, none, lo0, hi, dp, dred, tau, z);
  *tau_o = tau;
  *z_o = z;
  if (!gather) return;
  Gather<T, DIM> ga = make_gather<T, DIM>(&sm.ga, scan_scratch, dp, ra, tau, z);
#pragma unroll 1
  for (int c = 0; c < src.nc; ++c) {
    const Segs sg = chunk_segs(src.off, src.start, src.moff, src.mst, src.s_rec, src.ntab, src.N, src.nc, c);
    gather_entries<T, DIM>(ga, sg, ws, true);
    if (wrow) write_weights(sg, ws, wrow, tau, z, dp, true);
  }
  ga.finish(ra.out + (size_t)r * DIM, false);
}

// tau and z over the nC <= kCand candidates in LDS (one wave, or the sparsemax
// sort form), then their support gather and the row's output
template <typename T, int DIM>
__device__ __forceinline__ void finish_lds(const DecodeParams &dp, const RowsArgs &ra, int r, RowsLds<T, DIM> &sm,
                                           int nC, double mx, double Lb, double *dred, int *scan_scratch,
                                           double *s_tau, int *s_kstar, double *tau_o, double *z_o) {
  const int tid = threadIdx.x;
  double tau, z;
  const Above none{0.0, 0.0, 0.0, 0.0, 0.0};
  const double hi = mx - pow_neg_a((double)max(nC, 1), dp);  // F(hi) <= 1: at most nC entries above it
  if (dp.ibeta == 1 && dp.tau_method == 1) {
    tau = sparsemax_tau_sort(sm.lead.cx, nC, sm.lead.sortbuf, dred, s_kstar);
    double zz = 0.0;
    for (int i = tid; i < nC; i += kDThreads) {
      const double y = sm.lead.cx[i] - tau;
      if (y > 0.0) zz += y;
    }
    z = block_sum(zz, dred);
  } else {
    if (tid < kWave) {
      double t, zk = 0.0;
      const LdsVals src{sm.lead.cx, nC, tid, kWave};
      if (dp.ibeta == 2) t = newton_tau<2, LdsVals, WaveRed>(src, none, Lb, hi, dp, dred, &zk);
      else if (dp.ibeta == 1) t = newton_tau<1, LdsVals, WaveRed>(src, none, Lb, hi, dp, dred, &zk);
      else t = newton_tau<0, LdsVals, WaveRed>(src, none, Lb, hi, dp, dred, &zk);
      if (zk == 0.0) {  // F at t from the candidates
        double zz = 0.0;
        src.each([&](double x) { const double y = x - t; if (y > 0.0) zz += pw_rt(y, dp); });
        zk = wave_sum(zz);
      }
      if (tid == 0) {
        s_tau[0] = t;
        s_tau[1] = zk;
      }
    }
    __syncthreads();
    tau = s_tau[0];
    z = s_tau[1];
  }
  EKV_MARK(1, 4);
  if (tid == 0 && ra.tau) ra.tau[r] = tau / dp.a;
  Gather<T, DIM> ga = make_gather<T, DIM>(&sm.lead.ga, scan_scratch, dp, ra, tau, z);
#pragma unroll 1
  for (int k0 = 0; k0 < nC; k0 += 4 * kDThreads) {
    double x4[4];
    uint32_t t4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = k0 + 4 * tid + u;
      x4[u] = k < nC ? sm.lead.cx[k] : -INFINITY;
      t4[u] = k < nC ? sm.lead.cv[k] : 0u;
    }
    ga.template offer<4>(x4, t4);
  }
  ga.finish(ra.out + (size_t)r * DIM, false);
  *tau_o = tau;
  *z_o = z;
}

// The end of a row whose entries (at most 16 per thread, -inf for unused or
// dropped slots) are in registers: the candidates X > Lb in index order into
// LDS, tau and z (over LDS, or the block over the registers), then the
// support gather, the output and weights_out.
template <typename T, int DIM>
__device__ __forceinline__ void row_finish(const DecodeParams &dp, const RowsArgs &ra, int r, RowsLds<T, DIM> &sm,
                                           double (&xv)[16], const uint32_t (&tv)[16], const uint32_t (&lv)[16],
                                           double mx, double Lb, float *wrow, double *dred, int *scan_scratch,
                                           double *s_tau, int *s_kstar) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 16; ++u)
    if (!(xv[u] > Lb)) xv[u] = -INFINITY;
  int nC;
  {
    int mine = 0;
#pragma unroll
    for (int u = 0; u < 16; ++u) mine += xv[u] > Lb ? 1 : 0;
    int at = block_excl_scan(mine, scan_scratch, &nC);
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (xv[u] > Lb) {
        if (at < kCand) {
          sm.lead.cx[at] = xv[u];
          sm.lead.cv[at] = tv[u];
        }
        ++at;
      }
    __syncthreads();
  }
  EKV_MARK(1, 3);
  double tau, z;
  if (nC <= kCand) {
    finish_lds<T, DIM>(dp, ra, r, sm, nC, mx, Lb, dred, scan_scratch, s_tau, s_kstar, &tau, &z);
  } else {
    const Above none{0.0, 0.0, 0.0, 0.0, 0.0};
    const double hi = mx - pow_neg_a((double)nC, dp);
    solve_block(RegVals16{xv}, none, Lb, hi, dp, dred, tau, z);
    EKV_MARK(1, 4);
    if (tid == 0 && ra.tau) ra.tau[r] = tau / dp.a;
    Gather<T, DIM> ga = make_gather<T, DIM>(&sm.lead.ga, scan_scratch, dp, ra, tau, z);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      double x8[8];
      uint32_t t8[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        x8[u] = xv[8 * half + u];
        t8[u] = tv[8 * half + u];
      }
      ga.template offer<8>(x8, t8);
    }
    ga.finish(ra.out + (size_t)r * DIM, false);
  }
  if (wrow)
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const double y = xv[u] - tau;
      if (y > 0.0) wrow[lv[u]] = (float)(pw_rt(y, dp) / z);
    }
  EKV_MARK(1, 5);
}

// The blocks of a row.  Every block reads every slice's summary (entry
// counts, max and min) and builds the row's table of non-empty slices; the
// row has nc chunks (one when N <= kChunkCap, else about N / kChunkEnt, at
// most nh), a slice going to chunk floor(entries before it * nc / N); a block
// whose chunk index is nc or more leaves.  Each chunk counts its entries
// above mx - 2^-i (a certified bound Lc for the row: C entries above mx - d
// give F(mx - d - C^-(alpha-1)) >= 1).  A lone chunk holding the whole row
// in registers finishes it at once.  Otherwise a chunk of a row of at most
// kLargeN entries compacts its entries above Lc in place, and in a larger row
// adds its entries to the row's integer histogram instead.  The row's last
// chunk to arrive merges: the row bound Lb from every chunk's bound and the
// summed counts; a smaller row is solved and gathered there (one wave over
// LDS candidates, or the block).  In a large row the last chunk certifies a
// window [e_lo, e_hi] for tau from the histogram (bounds of F at the bin
// edges) and every chunk then (a) sums the moments of its entries above e_hi
// and hands over those in the window (the last to arrive solves for tau
// exactly) and (b) gathers its support (the last sums the partial outputs in
// chunk order).  Between (a) and (b) the chunks of a row wait for its last
// block; a row has at most nh <= 32 chunks, fewer than an XCD holds at once,
// and blocks are dispatched in index order, so every waited-for block is
// running.  Every decision and every sum depends on the entries alone, not on
// timing.
constexpr int kChunkPer = 16;                     // entries per thread a chunk block holds
constexpr int kChunkCap = kChunkPer * kDThreads;  // entries a chunk compacts
constexpr int kChunkEnt = 3072;                   // entries per chunk a split row aims at (slack for slice sizes)
constexpr int kMidCap = 16384;                    // entries a lone block streams over (two passes)
constexpr int kLastCap = 4096;                    // entries the last block solves over
constexpr int kSumPer = kMaxSlices / kDThreads;   // slice summaries per thread

template <typename T, int DIM>
__device__ __forceinline__ void row_block(const Dims &D, const DecodeParams &dp, const RowsArgs &ra, const DecodeWs &ws,
                                          int r, int c, RowsLds<T, DIM> &sm) {
  __shared__ double dred[3 * kDThreads / kWave];
  __shared__ int scan_scratch[kDThreads / kWave];
  __shared__ unsigned long long scan64[kDThreads / kWave];
  __shared__ int s_cnt[kDThreads / kWave][kNThr];
  __shared__ int s_nan[kDThreads / kWave];
  __shared__ double s_tau[2];
  __shared__ int s_kstar, s_last, s_ovf;
  __shared__ unsigned s_flag;
  __shared__ double s_rec[kHelpers][13];
  __shared__ double s_par[8];
  __shared__ double s_hp[kHelpers][5];
  __shared__ int s_woff[kHelpers + 1];
  __shared__ double s_amin;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int ns = ra.ns;
  float *wrow = ra.weights_out ? ra.weights_out + (size_t)r * D.max_pages * D.P : nullptr;
  EKV_MARK(1, 0);
  if (c > 0) {  // a chunk index past the row's bound on chunks (from its items) leaves at once
    const long long ub = (long long)ws.rcnt[r] * D.P;
    if (ub <= kMidCap || c >= (int)((ub + kChunkEnt - 1) / kChunkEnt)) return;
  }
  // 1. the slices' summaries: the row's max, min and malformed mark (one
  // barrier), then the table of the slices holding entries above mx - 1 (one
  // packed scan: table position high, entry offset low).  A slice whose max
  // is at most mx - 1 holds no entry that can carry weight (tau >= mx - 1).
  const int per = (ns + kDThreads - 1) / kDThreads;
  const int i0 = tid * per;
  int scn[kSumPer];
  uint32_t sst[kSumPer];
  double smx[kSumPer];
  double mx = -INFINITY, mn = INFINITY;
  int nan = 0;
#pragma unroll
  for (int u = 0; u < kSumPer; ++u) {
    scn[u] = 0;
    smx[u] = -INFINITY;
    const int i = i0 + u;
    if (u < per && i < ns) {
      const size_t o = (size_t)r * ns + i;
      scn[u] = ws.s_cnt[o];
      sst[u] = ws.s_start[o];
      smx[u] = ws.s_max[o];
      nan |= smx[u] != smx[u];
      mx = fmax(mx, smx[u]);
      mn = fmin(mn, ws.s_min[o]);
    }
  }
  {
    const double wmx = wave_max(mx), wmn = wave_min_d(mn);
    const int wnan = __any(nan) ? 1 : 0;
    if (lane == 0) {
      dred[wv] = wmx;
      dred[kDThreads / kWave + wv] = wmn;
      s_nan[wv] = wnan;
    }
    __syncthreads();
    mx = dred[0];
    mn = dred[kDThreads / kWave];
    nan = s_nan[0];
    for (int i = 1; i < kDThreads / kWave; ++i) {
      mx = fmax(mx, dred[i]);
      mn = fmin(mn, dred[kDThreads / kWave + i]);
      nan |= s_nan[i];
    }
  }
  const double thr = mx - 1.0;  // tau >= thr: F(mx - 1) >= 1
  unsigned long long mine = 0;
#pragma unroll
  for (int u = 0; u < kSumPer; ++u) {
    if (!(smx[u] > thr)) scn[u] = 0;
    if (scn[u] > 0) mine += (1ull << 32) + (unsigned)scn[u];
  }
  {
    unsigned long long tot;
    unsigned long long run = block_excl_scan64(mine, scan64, &tot);
#pragma unroll
    for (int u = 0; u < kSumPer; ++u) {
      const int i = i0 + u;
      if (u < per && i < ns && scn[u] > 0) {
        const int at = (int)(run >> 32);
        sm.off[at] = (int)(run & 0xFFFFFFFFull);
        sm.start[at] = sst[u];
        run += (1ull << 32) + (unsigned)scn[u];
      }
    }
    mine = tot;
  }
  const int ntab = (int)(mine >> 32), N = (int)(mine & 0xFFFFFFFFull);
  if (tid == 0) sm.off[ntab] = N;
  __syncthreads();
  const int nc = N > kMidCap ? min(ra.nh, (N + kChunkEnt - 1) / kChunkEnt) : 1;
  if (c >= nc) return;
  const bool large = N > kLargeN && dp.ibeta != 0;
  int t0, t1;
  chunk_window(sm.off, ntab, N, nc, c, &t0, &t1);
  const Segs sg = segs_window(sm.off, sm.start, t0, t1);
  const int M = sg.total;
  EKV_MARK(1, 6);
  // histogram range of a large row: every entry above lo is binned
  double hlo = fmax(thr, mn);
  double hw = (mx - hlo) / (double)kBins;
  if (!(hw > 0.0) || !(hw < INFINITY)) hw = 1.0 / (double)kBins;
  // bins by a product with 1/w: its rounding moves an entry by at most one
  // bin, which the window's bounds allow for (a bin's entries are taken to lie
  // anywhere in the bins beside it)
  const double inv_hw = 1.0 / hw;
  if (nc == 1 && !large && M > kChunkCap) {
    // a lone block over more entries than its registers hold: rounds of
    // kChunkCap entries (16 per thread).  The counts of the rounds so far
    // already certify a bound (a part of the row's entries gives a weaker
    // one), so each round puts its entries above the bound reached into the
    // LDS candidates (a fixed order) and the entries are read once.
    if (nan) {
      row_nan<DIM>(ra, r);
      return;
    }
    int q8[kNThr];
#pragma unroll
    for (int i = 0; i < kNThr; ++i) q8[i] = 0;
    double Lq = thr;
    int nC = 0;
    const int rounds = (M + kChunkCap - 1) / kChunkCap;
#pragma unroll 1
    for (int qr = 0; qr < rounds; ++qr) {
      double xq[kChunkPer];
      uint32_t tq[kChunkPer];
      {
        size_t ad[kChunkPer];
        addr_strided<kChunkPer>(sg, qr * kChunkCap + tid, ad);
#pragma unroll
        for (int u = 0; u < kChunkPer; ++u) {
          xq[u] = ws.cx[ad[u]];
          tq[u] = ws.ct[ad[u]];
        }
      }
#pragma unroll
      for (int u = 0; u < kChunkPer; ++u) {
        if (qr * kChunkCap + tid + u * kDThreads >= M) xq[u] = -INFINITY;
        if (xq[u] > thr)
#pragma unroll
          for (int i = 0; i < kNThr; ++i) q8[i] += xq[u] > mx - ldexp(1.0, -i) ? 1 : 0;
      }
      {
        int w8[kNThr];
#pragma unroll
        for (int i = 0; i < kNThr; ++i) w8[i] = wave_sum(q8[i]);
        if (lane == 0)
          for (int i = 0; i < kNThr; ++i) s_cnt[wv][i] = w8[i];
        __syncthreads();
        const int i = tid & (kNThr - 1);
        int ci_ = 0;
        for (int w = 0; w < kDThreads / kWave; ++w) ci_ += s_cnt[w][i];
        const double cand =
            ci_ > 0 ? (mx - ldexp(1.0, -i)) - pow_neg_a((double)ci_, dp) - 1e-12 * fmax(1.0, fabs(mx)) : -INFINITY;
        Lq = fmax(Lq, wave_max(cand));
      }
      int take = 0;
#pragma unroll
      for (int u = 0; u < kChunkPer; ++u) take += xq[u] > Lq ? 1 : 0;
      int tot;
      int at = nC + block_excl_scan(take, scan_scratch, &tot);
#pragma unroll
      for (int u = 0; u < kChunkPer; ++u)
        if (xq[u] > Lq) {
          if (at < kCand) {
            sm.lead.cx[at] = xq[u];
            sm.lead.cv[at] = tq[u];
          }
          ++at;
        }
      nC += tot;
    }
    __syncthreads();
    EKV_MARK(1, 3);
    double tau, z;
    if (nC <= kCand) {
      finish_lds<T, DIM>(dp, ra, r, sm, nC, mx, Lq, dred, scan_scratch, s_tau, &s_kstar, &tau, &z);
    } else {  // many candidates: passes over the row's entries
      if (tid == 0) s_rec[0][11] = 0.0;
      __syncthreads();
      const RowVals rv{&ws, sm.off, sm.moff, sm.start, sm.mst, s_rec, ntab, N, 1};
      row_slow<T, DIM>(dp, ra, ws, r, sm, rv, Lq, mx, dred, scan_scratch, nullptr, true, &tau, &z);
      if (tid == 0 && ra.tau) ra.tau[r] = tau / dp.a;
    }
    if (wrow) write_weights(sg, ws, wrow, tau, z, dp, false);
    EKV_MARK(1, 5);
    return;
  }
  // 2. counts above mx - 2^-i; compaction (smaller rows) or histogram (large)
  int c8[kNThr];
#pragma unroll
  for (int i = 0; i < kNThr; ++i) c8[i] = 0;
  auto count1 = [&](double x) __attribute__((always_inline)) {
    if (x > thr)
#pragma unroll
      for (int i = 0; i < kNThr; ++i) c8[i] += x > mx - ldexp(1.0, -i) ? 1 : 0;
  };
  const bool small = !large && M <= kChunkCap;
  double xv[kChunkPer];
  uint32_t tv[kChunkPer], lv[kChunkPer];
  if (large)
    for (int i = tid; i < kBins; i += kDThreads) sm.hist[i] = 0u;
  if (large) __syncthreads();
  if (!nan && M > 0) {
    if (small) {
      // entries tid + u * kDThreads (a fixed order of the chunk's entries)
      size_t ad[kChunkPer];
      addr_strided<kChunkPer>(sg, tid, ad);
      EKV_MARK(3, 0);
#pragma unroll
      for (int u = 0; u < kChunkPer; ++u) {
        xv[u] = ws.cx[ad[u]];
        tv[u] = ws.ct[ad[u]];
        lv[u] = wrow ? ws.cl[ad[u]] : 0u;
      }
#pragma unroll
      for (int u = 0; u < kChunkPer; ++u) {
        if (tid + u * kDThreads >= M) xv[u] = -INFINITY;
        count1(xv[u]);
      }
      EKV_MARK(3, 1);
    } else {
      stream_batches(sg, ws, false, false, [&](const Batch8 &bt) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const double x = bt.v[u];
          count1(x);
          if (large && x > hlo) {
            const double f = floor((x - hlo) * inv_hw);
            const int bin = !(f >= 0.0) ? 0 : (f >= (double)kBins ? kBins - 1 : (int)f);
            atomicAdd(&sm.hist[bin], 1u);
          }
        }
      });
    }
  } else {
#pragma unroll
    for (int u = 0; u < kChunkPer; ++u) {
      xv[u] = -INFINITY;
      tv[u] = 0u;
      lv[u] = 0u;
    }
  }
#pragma unroll
  for (int i = 0; i < kNThr; ++i) c8[i] = wave_sum(c8[i]);
  if (lane == 0)
    for (int i = 0; i < kNThr; ++i) s_cnt[wv][i] = c8[i];
  __syncthreads();
  EKV_MARK(3, 2);
  if (large)
    for (int i = tid; i < kBins; i += kDThreads)
      if (sm.hist[i]) atomicAdd(&ws.hist[(size_t)r * kBins + i], sm.hist[i]);
  double Lc;
  {
    const int i = tid & (kNThr - 1);
    int ci_ = 0;
    for (int w = 0; w < kDThreads / kWave; ++w) ci_ += s_cnt[w][i];
    const double cand =
        ci_ > 0 ? (mx - ldexp(1.0, -i)) - pow_neg_a((double)ci_, dp) - 1e-12 * fmax(1.0, fabs(mx)) : -INFINITY;
    Lc = fmax(thr, wave_max(cand));  // every wave holds the same counts
  }
  EKV_MARK(1, 7);
  if (nc == 1 && small) {
    // a lone chunk holds the whole row in registers: the candidates above Lb
    // (= Lc, the row's own counts) go to LDS directly
    if (nan) row_nan<DIM>(ra, r);
    else if (N == 0) row_empty<DIM>(ra, r);
    else row_finish<T, DIM>(dp, ra, r, sm, xv, tv, lv, mx, Lc, wrow, dred, scan_scratch, s_tau, &s_kstar);
    return;
  }
  const uint32_t cstart = t1 > t0 ? sm.start[t0] : 0u;  // the chunk's first entry position
  int m = M;
  if (small && !nan && M > 0) {
    // in place: every entry of the chunk is in registers before the scan's
    // barrier, and the m kept ones go to [cstart, cstart + m), inside the
    // chunk's own slice regions (which follow each other from cstart and
    // hold at least its M entries)
    int mineC = 0;
#pragma unroll
    for (int u = 0; u < kChunkPer; ++u) mineC += xv[u] > Lc ? 1 : 0;
    int at = block_excl_scan(mineC, scan_scratch, &m);
#pragma unroll
    for (int u = 0; u < kChunkPer; ++u)
      if (xv[u] > Lc) {
        st_agent(&ws.cx[cstart + at], xv[u]);
        st_agent(&ws.ct[cstart + at], tv[u]);
        if (wrow) st_agent(&ws.cl[cstart + at], lv[u]);
        ++at;
      }
  }
  if (tid == 0) {
    double *rec = ws.crec + ((size_t)r * kHelpers + c) * 16;
    st_agent(&rec[0], (double)m);
    st_agent(&rec[1], Lc);
    for (int i = 0; i < kNThr; ++i)
      st_agent(&rec[2 + i], (double)(s_cnt[0][i] + s_cnt[1][i] + s_cnt[2][i] + s_cnt[3][i]));
    st_agent(&rec[10], (double)cstart);
    st_agent(&rec[11], small ? 1.0 : 0.0);
    st_agent(&rec[12], (double)M);
  }
  EKV_MARK(1, 1);
  if (nc > 1 && !arrive_last(&ws.ctr[4 * r + 3], (unsigned)nc, &s_last)) {
    if (!large) return;
  } else {
    // ---- 3. the row's last chunk: merge (a lone chunk first completes its
    // own record and histogram stores)
    EKV_MARK(1, 2);
    if (nc == 1) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    if (tid < nc) {  // all of a record's fields requested at once (one round trip)
      double v[13];
#pragma unroll
      for (int f = 0; f < 13; ++f) v[f] = ld_agent(&ws.crec[((size_t)r * kHelpers + tid) * 16 + f]);
#pragma unroll
      for (int f = 0; f < 13; ++f) s_rec[tid][f] = v[f];
    }
    __syncthreads();
    if (nan || N == 0) {
      if (nan) row_nan<DIM>(ra, r);
      else row_empty<DIM>(ra, r);
      if (large) publish_step(&ws.state[(size_t)r * kStStride], kStDone);
      return;
    }
    int mtot = 0;
    bool all_small = true;
    for (int cc = 0; cc < nc; ++cc) {
      mtot += (int)s_rec[cc][0];
      all_small &= s_rec[cc][11] != 0.0;
    }
    if (tid == 0) {  // the compacted runs
      int o = 0;
      for (int cc = 0; cc < nc; ++cc) {
        sm.moff[cc] = o;
        sm.mst[cc] = (uint32_t)s_rec[cc][10];
        if (s_rec[cc][11] != 0.0) o += (int)s_rec[cc][0];
      }
      sm.moff[nc] = o;
    }
    double Lb;
    {
      // lane i (mod kNThr): threshold i's bound from the summed counts
      const int i = tid & (kNThr - 1);
      int ct = 0;
      for (int cc = 0; cc < nc; ++cc) ct += (int)s_rec[cc][2 + i];
      const double cand =
          ct > 0 ? (mx - ldexp(1.0, -i)) - pow_neg_a((double)ct, dp) - 1e-12 * fmax(1.0, fabs(mx)) : -INFINITY;
      double bnd = wave_max(cand);
      for (int cc = 0; cc < nc; ++cc) bnd = fmax(bnd, s_rec[cc][1]);
      Lb = fmax(thr, bnd);
    }
    __syncthreads();  // the runs table
    const RowVals rv{&ws, sm.off, sm.moff, sm.start, sm.mst, s_rec, ntab, N, nc};
    if (large) {
      // ---- certified window from the row's histogram.  Bin b's entries lie
      // in [e_{b-1}, e_{b+2}] (one bin of slack for the rounding of the
      // binning), so
      //   LB(k) = sum_{b >= k+2} n_b ((b-1-k) w)^beta <= F(e_k)
      //   UB(k) = sum_{b >= k-1} n_b ((b+2-k) w)^beta >= F(e_k)
      // (entries at or below lo add nothing at an edge e_k >= lo), written
      // with suffix sums of n_b, n_b b, n_b b^2 in integers.  tau lies in
      // [e_klo, e_khi]: klo the largest edge with LB >= 1 (else Lb), khi the
      // smallest with UB <= 1 (1 -/+ 1e-9 for the final rounding).
      for (int i = tid; i < kBins; i += kDThreads) sm.hist[i] = ld_agent(&ws.hist[(size_t)r * kBins + i]);
      __syncthreads();
      constexpr int kPer = kBins / kDThreads;
      long long l0 = 0, l1 = 0, l2 = 0;
      for (int u = 0; u < kPer; ++u) {
        const long long bb = (long long)tid * kPer + u, n = sm.hist[bb];
        l0 += n;
        l1 += n * bb;
        l2 += n * bb * bb;
      }
      unsigned long long t0_, t1_, t2_;
      const long long q0 = (long long)block_excl_scan64((unsigned long long)l0, scan64, &t0_);
      const long long q1 = (long long)block_excl_scan64((unsigned long long)l1, scan64, &t1_);
      const long long q2 = (long long)block_excl_scan64((unsigned long long)l2, scan64, &t2_);
      long long S0 = (long long)t0_ - q0, S1 = (long long)t1_ - q1, S2 = (long long)t2_ - q2;
      const double wb = dp.ibeta == 2 ? hw * hw : hw;
      int klo = -1, khi = 0x7fffffff;
      auto nb = [&](long long bb) -> long long { return (bb >= 0 && bb < kBins) ? (long long)sm.hist[bb] : 0ll; };
      const int kend = tid == kDThreads - 1 ? kPer + 1 : kPer;  // the last thread also takes edge kBins
      for (int u = 0; u < kend; ++u) {
        const long long k = (long long)tid * kPer + u;
        const long long a0 = nb(k), a1 = nb(k + 1);
        const long long T0 = S0 - a0 - a1, T1 = S1 - a0 * k - a1 * (k + 1);
        const long long T2 = S2 - a0 * k * k - a1 * (k + 1) * (k + 1);
        const long long mm = k > 0 ? k - 1 : 0, am = k > 0 ? nb(k - 1) : 0;
        const long long U0 = S0 + am, U1 = S1 + am * mm, U2 = S2 + am * mm * mm;
        double lb, ub;
        if (dp.ibeta == 2) {
          lb = (double)(T2 - 2 * (k + 1) * T1 + (k + 1) * (k + 1) * T0) * wb;
          ub = (double)(U2 + 2 * (2 - k) * U1 + (2 - k) * (2 - k) * U0) * wb;
        } else {
          lb = (double)(T1 - (k + 1) * T0) * wb;
          ub = (double)(U1 + (2 - k) * U0) * wb;
        }
        if (lb >= 1.0 + 1e-9) klo = max(klo, (int)k);
        if (ub <= 1.0 - 1e-9) khi = min(khi, (int)k);
        S0 -= a0;
        S1 -= a0 * k;
        S2 -= a0 * k * k;
      }
      klo = (int)block_max((double)klo, dred);
      khi = (int)block_min_d((double)khi, dred);
      if (tid == 0) {
        const double e_lo = fmax(klo >= 0 ? hlo + (double)klo * hw : Lb, Lb);
        const double e_hi = khi <= kBins ? hlo + (double)khi * hw : mx;
        st_agent(&ws.rpar[(size_t)r * 8 + 3], e_lo);
        st_agent(&ws.rpar[(size_t)r * 8 + 4], fmax(e_hi, e_lo));
      }
      EKV_MARK(1, 3);
      publish_step(&ws.state[(size_t)r * kStStride], kStMom);
    } else if (!all_small || mtot > kLastCap) {
      // many candidates: passes over the row's entries by this block
      double tau, z;
      row_slow<T, DIM>(dp, ra, ws, r, sm, rv, Lb, mx, dred, scan_scratch, wrow, true, &tau, &z);
      if (tid == 0 && ra.tau) ra.tau[r] = tau / dp.a;
      return;
    } else {
      // ---- the compacted entries (16 consecutive per thread), those above
      // Lb into LDS in index order, then tau and the gather
      const Segs cs = segs_window(sm.moff, sm.mst, 0, nc);
      {
        size_t ad[kChunkPer];
        if (mtot > 0) addr_strided<kChunkPer>(cs, tid, ad);
#pragma unroll
        for (int u = 0; u < kChunkPer; ++u) {
          const bool in = tid + u * kDThreads < mtot;
          xv[u] = in ? ld_agent(&ws.cx[ad[u]]) : -INFINITY;
          tv[u] = in ? ld_agent(&ws.ct[ad[u]]) : 0u;
          lv[u] = (in && wrow) ? ld_agent(&ws.cl[ad[u]]) : 0u;
        }
      }
      row_finish<T, DIM>(dp, ra, r, sm, xv, tv, lv, mx, Lb, wrow, dred, scan_scratch, s_tau, &s_kstar);
      return;
    }
  }
  // ---- large row, every chunk: (a) moments above e_hi and the window entries
  if (wait_step(&ws.state[(size_t)r * kStStride], kStMom, &s_flag) != kStMom) {
    if (s_flag == 0u) row_nan<DIM>(ra, r);  // time limit
    return;
  }
  EKV_MARK(2, 0);
  if (tid < 8) s_par[tid] = ld_agent(&ws.rpar[(size_t)r * 8 + tid]);
  __syncthreads();
  const double e_lo = s_par[3], e_hi = s_par[4];
  {
    double m1 = 0.0, m2 = 0.0, ymin = INFINITY;
    int m0 = 0, wc = 0;
    double *slot = ws.wbuf + ((size_t)r * kHelpers + c) * kSlot;
    stream_batches(sg, ws, false, false, [&](const Batch8 &bt) __attribute__((always_inline)) {
      int take = 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const double v = bt.v[u];
        if (v > e_hi) {
          const double y = v - e_hi;
          ++m0;
          m1 += y;
          m2 += y * y;
          ymin = fmin(ymin, y);
        } else if (v > e_lo) {
          ++take;
        }
      }
      int tot;
      int at = wc + block_excl_scan<true>(take, scan_scratch, &tot);  // the next batch's loads stay in flight
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (!(bt.v[u] > e_hi) && bt.v[u] > e_lo) {
          if (at < kSlot) st_agent(&slot[at], bt.v[u]);
          ++at;
        }
      wc += tot;
    });
    double sums[3] = {(double)m0, m1, m2};
    block_sum_n<3>(sums, dred);
    ymin = block_min_d(ymin, dred);
    if (tid == 0) {
      double *hp = ws.hpart + ((size_t)r * kHelpers + c) * 8;
      st_agent(&hp[0], sums[0]);
      st_agent(&hp[1], sums[1]);
      st_agent(&hp[2], sums[2]);
      st_agent(&hp[3], ymin);
      st_agent(&hp[4], (double)wc);
    }
  }
  if (arrive_last(&ws.ctr[4 * r + 1], (unsigned)nc, &s_last)) {
    // the row's last: tau from the moments and the window entries
    if (tid < nc) {
      double v[5];
#pragma unroll
      for (int f = 0; f < 5; ++f) v[f] = ld_agent(&ws.hpart[((size_t)r * kHelpers + tid) * 8 + f]);
#pragma unroll
      for (int f = 0; f < 5; ++f) s_hp[tid][f] = v[f];
    }
    __syncthreads();
    if (tid == 0) {
      double a0 = 0.0, a1 = 0.0, a2 = 0.0, amin = INFINITY;
      int off = 0, ovf = 0;
      for (int h = 0; h < nc; ++h) {
        a0 += s_hp[h][0];
        a1 += s_hp[h][1];
        a2 += s_hp[h][2];
        amin = fmin(amin, s_hp[h][3]);
        s_woff[h] = off;
        const int cnt_h = (int)s_hp[h][4];
        ovf |= cnt_h > kSlot ? 1 : 0;
        off += cnt_h;
      }
      s_woff[nc] = off;
      s_ovf = ovf | (off > kWin ? 1 : 0);
      s_par[5] = a0;
      s_par[6] = a1;
      s_par[7] = a2;
      s_amin = amin;
    }
    __syncthreads();
    const Above ab{s_par[5], s_par[6], s_par[7], s_amin, e_hi};
    const int W = s_woff[nc];
    const bool ovf = s_ovf != 0;
    double tau, z;
    if (!ovf) {
      for (int h = 0; h < nc; ++h) {
        const int n = s_woff[h + 1] - s_woff[h];
        for (int i = tid; i < n; i += kDThreads)
          sm.win[s_woff[h] + i] = ld_agent(&ws.wbuf[((size_t)r * kHelpers + h) * kSlot + i]);
      }
      __syncthreads();
      solve_block(LdsVals{sm.win, W, tid, kDThreads}, ab, e_lo, e_hi, dp, dred, tau, z);
    } else {
      // window too wide for the slots: passes over every entry of the row
      // (every chunk of a large row is in place: the row's table)
      if (tid == 0) {
        for (int cc = 0; cc < nc; ++cc) s_rec[cc][11] = 0.0;
      }
      __syncthreads();
      const RowVals rv{&ws, sm.off, sm.moff, sm.start, sm.mst, s_rec, ntab, N, nc};
      row_slow<T, DIM>(dp, ra, ws, r, sm, rv, e_lo, e_hi, dred, scan_scratch, nullptr, false, &tau, &z);
    }
    if (tid == 0) {
      st_agent(&ws.rpar[(size_t)r * 8 + 5], tau);
      st_agent(&ws.rpar[(size_t)r * 8 + 6], z);
      if (ra.tau) ra.tau[r] = tau / dp.a;
    }
    EKV_MARK(2, 1);
    publish_step(&ws.state[(size_t)r * kStStride], kStGath);
  }
  // ---- (b) the support gather of this chunk; the last sums the partial
  // outputs in chunk order
  if (wait_step(&ws.state[(size_t)r * kStStride], kStGath, &s_flag) != kStGath) {
    if (s_flag == 0u) row_nan<DIM>(ra, r);
    return;
  }
  if (tid < 8) s_par[tid] = ld_agent(&ws.rpar[(size_t)r * 8 + tid]);
  __syncthreads();
  Gather<T, DIM> ga = make_gather<T, DIM>(&sm.ga, scan_scratch, dp, ra, s_par[5], s_par[6]);
  gather_entries<T, DIM>(ga, sg, ws, false);
  ga.finish(ws.opart + ((size_t)r * kHelpers + c) * DIM, true);
  if (wrow) write_weights(sg, ws, wrow, s_par[5], s_par[6], dp, false);
  if (!arrive_last(&ws.ctr[4 * r + 2], (unsigned)nc, &s_last)) return;
  for (int cc = tid; cc < DIM; cc += kDThreads) {
    // every chunk's partial requested at once, then added in chunk order
    float part[kHelpers];
#pragma unroll
    for (int h = 0; h < kHelpers; ++h)
      part[h] = h < nc ? ld_agent(&ws.opart[((size_t)r * kHelpers + h) * DIM + cc]) : 0.0f;
    float sum = part[0];
#pragma unroll
    for (int h = 1; h < kHelpers; ++h)
      if (h < nc) sum += part[h];
    ra.out[(size_t)r * DIM + cc] = sum;
  }
  EKV_MARK(2, 2);
  publish_step(&ws.state[(size_t)r * kStStride], kStDone);
}

// Block index: row r's blocks are r * nh .. r * nh + nh - 1.
template <typename T, int DIM>
__global__ __launch_bounds__(kDThreads) void rows_kernel(Dims D, DecodeParams dp, RowsArgs ra, DecodeWs ws) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  RowsLds<T, DIM> &sm = *reinterpret_cast<RowsLds<T, DIM> *>(smem_raw);
  const int rows = D.B * D.Hq;
  const int bid = blockIdx.x;
  if (bid < rows * ra.nh) row_block<T, DIM>(D, dp, ra, ws, bid / ra.nh, bid % ra.nh, sm);
}

// =================================================================== launchers
// Query-head rows up to which a set per query head goes to the per-item
// decode: there a step is a few dependent memory round trips per kernel, and
// one page per block in flight beats the slices' union step; above it the
// slices share each K page among the heads of a group and split large rows.
constexpr long long kItemRows = 64;

static int decode_slices(const Dims &D) {
  long long ns = (D.max_pages + 127) / 128;  // about 128 pages per slice
  ns = std::max(ns, (long long)((D.max_pages + kMaxR - 1) / kMaxR));
  ns = std::min(ns, (long long)std::max(1, D.max_pages));
  ns = std::min(ns, (long long)kMaxSlices);
  return (int)std::max(1ll, ns);
}

static DecodeWs carve_decode(const Dims &D, int ns, long long item_cap, void *base, size_t *bytes) {
  Carve cv(base);
  const size_t rows = (size_t)D.B * D.Hq, cap_tok = (size_t)item_cap * D.P;
  DecodeWs w;
  w.cx = cv.take<double>(cap_tok);
  w.ct = cv.take<uint32_t>(cap_tok);
  w.cl = cv.take<uint32_t>(cap_tok);
  w.s_cnt = cv.take<int>(rows * ns);
  w.s_max = cv.take<double>(rows * ns);
  w.s_min = cv.take<double>(rows * ns);
  w.s_start = cv.take<uint32_t>(rows * ns);
  w.rcnt = cv.take<int>(rows);
  w.state = cv.take<unsigned>(rows * kStStride);
  w.ctr = cv.take<unsigned>(rows * 4);
  w.rpar = cv.take<double>(rows * 8);
  w.crec = cv.take<double>(rows * kHelpers * 16);
  w.hist = cv.take<unsigned>(rows * kBins);
  w.hpart = cv.take<double>(rows * kHelpers * 8);
  w.wbuf = cv.take<double>(rows * kHelpers * kSlot);
  w.opart = cv.take<float>(rows * kHelpers * D.d);
  if (bytes) *bytes = cv.bytes();
  return w;
}

// item capacity limit: every row's full set, and tokens addressable in 32 bits
static long long cap_limit(const Dims &D) {
  const long long dense = (long long)D.B * D.Hq * D.max_pages;
  return std::min(dense, (long long)(0xFFFFFFFFll / D.P));
}

size_t decode_ws_bytes_items(const Dims &D, long long items) {
  size_t b = 0;
  carve_decode(D, decode_slices(D), std::min(std::max(items, 1ll), cap_limit(D)), nullptr, &b);
  return b;
}
size_t decode_ws_bytes(const Dims &D, bool) { return decode_ws_bytes_items(D, cap_limit(D)); }
size_t full_ws_bytes(const Dims &D) { return decode_ws_bytes(D, true); }
size_t decode_group_ws_bytes(const Dims &D) { return decode_ws_bytes(D, false); }
size_t decode_ws_min_bytes(const Dims &D) { return decode_ws_bytes_items(D, 1); }

// items a workspace of ws_bytes holds
static long long item_cap_of(const Dims &D, int ns, size_t ws_bytes) {
  size_t fixed = 0;
  carve_decode(D, ns, 0, nullptr, &fixed);
  if (ws_bytes <= fixed) return 0;
  // an upper estimate (the three token regions without their alignment), then
  // down to the largest capacity that fits: a few steps at most
  long long cap = (long long)((ws_bytes - fixed) / ((size_t)D.P * 16));
  cap = std::min(cap, cap_limit(D));
  size_t b = 0;
  carve_decode(D, ns, cap, nullptr, &b);
  while (cap > 0 && b > ws_bytes) {
    --cap;
    carve_decode(D, ns, cap, nullptr, &b);
  }
  return cap;
}

template <typename T, int DIM, int P, int G>
static hipError_t launch_dec_t(const Dims &D, const DecodeParams &dp, const KsArgs &ka, const void *v_pool, float *out,
                               double *tau, const DecodeWs &w, hipStream_t s) {
  const int groups = D.B * D.Hkv, rows = D.B * D.Hq;
  hipLaunchKernelGGL((scores_kernel<T, DIM, P, G>), dim3(groups * ka.ns), dim3(kDThreads), 0, s, D, dp, ka, w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  static bool attr_set = false;
  const size_t lds = sizeof(RowsLds<T, DIM>);
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void *)rows_kernel<T, DIM>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    attr_set = true;
  }
  // blocks per row (chunks at most).  A chunk of a large row holds its slot
  // while it waits for its row's last block, so more chunks per row leave fewer
  // rows in flight; measured on gfx950 (slice decode): 512 rows of 10^5 entries
  // 7 chunks 2.20 ms (1 chunk 3.12, 3 2.84, 15 2.30, 31 2.75), 32 rows of ~10^6
  // tokens (full cache) 15 chunks 504 us (7 541, 31 ~600).  Blocks past a row's
  // bound on chunks leave at once.  An odd count spreads the rows' first blocks
  // over the XCDs (blocks go to the XCDs in turn).
  const int nh = std::max(1, std::min(std::min(kHelpers - 1, ka.ns), rows >= 256 ? 7 : 15));
  RowsArgs ra{v_pool, out, tau, ka.weights_out, ka.ns, nh};
  const long long grid = (long long)rows * nh;
  hipLaunchKernelGGL((rows_kernel<T, DIM>), dim3((unsigned)grid), dim3(kDThreads), lds, s, D, dp, ra, w);
  return hipGetLastError();
}

template <typename T, int DIM, int P>
static hipError_t launch_dec_g(const Dims &D, const DecodeParams &dp, const KsArgs &ka, const void *v, float *out,
                               double *tau, const DecodeWs &w, hipStream_t s) {
  switch (D.G) {
    case 1: return launch_dec_t<T, DIM, P, 1>(D, dp, ka, v, out, tau, w, s);
    case 2: return launch_dec_t<T, DIM, P, 2>(D, dp, ka, v, out, tau, w, s);
    case 4: return launch_dec_t<T, DIM, P, 4>(D, dp, ka, v, out, tau, w, s);
    case 8: return launch_dec_t<T, DIM, P, 8>(D, dp, ka, v, out, tau, w, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, int DIM>
static hipError_t launch_dec_p(const Dims &D, const DecodeParams &dp, const KsArgs &ka, const void *v, float *out,
                               double *tau, const DecodeWs &w, hipStream_t s) {
  if (D.P == 16) return launch_dec_g<T, DIM, 16>(D, dp, ka, v, out, tau, w, s);
  if (D.P == 32) return launch_dec_g<T, DIM, 32>(D, dp, ka, v, out, tau, w, s);
  return launch_dec_g<T, DIM, 64>(D, dp, ka, v, out, tau, w, s);
}

// mode: 0 a set per query head, 1 a set per KV head, 2 every page
static hipError_t launch_decode_mode(const Dims &D, int dtype, int mode, const void *q, const void *k_pool,
                                     const void *v_pool, const int32_t *page_table, const int32_t *seq_lens,
                                     const int32_t *sel_idx, const int32_t *sel_cnt, double alpha, int tau_method,
                                     float *out, double *tau, float *weights_out, void *ws, size_t ws_bytes,
                                     hipStream_t s) {
  DecodeParams dp;
  dp.a = alpha - 1.0;
  dp.beta = 1.0 / dp.a;
  dp.c = D.scale;
  dp.ibeta = alpha == 1.5 ? 2 : (alpha == 2.0 ? 1 : 0);
  dp.tau_method = tau_method;
  const int ns = decode_slices(D);
  if ((D.max_pages + ns - 1) / ns > kMaxR) return hipErrorInvalidValue;
  // an entry's V row (physical page * Hkv + g) * P + slot is held in 32 bits
  if ((unsigned long long)D.num_phys * (unsigned long long)D.Hkv * (unsigned long long)D.P > 0xFFFFFFFFull)
    return hipErrorInvalidValue;
  const long long cap = item_cap_of(D, ns, ws_bytes);
  // a set per query head over a few rows: the per-item decode (decode_items.hip),
  // same item capacity (its layout needs fewer bytes per item)
  if (mode == 0 && (long long)D.B * D.Hq <= kItemRows && decode_items_ws_bytes(D, cap) <= ws_bytes)
    return launch_entmax_decode_items(D, dtype, q, k_pool, v_pool, page_table, seq_lens, sel_idx, sel_cnt, alpha,
                                      tau_method, out, tau, weights_out, ws, cap, s);
  const DecodeWs w = carve_decode(D, ns, cap, ws, nullptr);
  const KsArgs ka{q, k_pool, page_table, seq_lens, sel_idx, sel_cnt, weights_out, mode, ns, cap};
  if (dtype == ENTMAXKV_BF16) {
    if (D.d == 64) return launch_dec_p<uint16_t, 64>(D, dp, ka, v_pool, out, tau, w, s);
    return launch_dec_p<uint16_t, 128>(D, dp, ka, v_pool, out, tau, w, s);
  }
  if (D.d == 64) return launch_dec_p<float, 64>(D, dp, ka, v_pool, out, tau, w, s);
  return launch_dec_p<float, 128>(D, dp, ka, v_pool, out, tau, w, s);
}

hipError_t launch_entmax_decode(const Dims &D, int dtype, const void *q, const void *k_pool, const void *v_pool,
                                const int32_t *page_table, const int32_t *seq_lens, const int32_t *sel_idx,
                                const int32_t *sel_cnt, double alpha, int tau_method, float *out, double *tau,
                                float *weights_out, void *ws, size_t ws_bytes, hipStream_t s) {
  return launch_decode_mode(D, dtype, 0, q, k_pool, v_pool, page_table, seq_lens, sel_idx, sel_cnt, alpha,
                            tau_method, out, tau, weights_out, ws, ws_bytes, s);
}

hipError_t launch_entmax_decode_group(const Dims &D, int dtype, const void *q, const void *k_pool,
                                      const void *v_pool, const int32_t *page_table, const int32_t *seq_lens,
                                      const int32_t *sel_idx, const int32_t *sel_cnt, double alpha, int tau_method,
                                      float *out, double *tau, float *weights_out, void *ws, size_t ws_bytes,
                                      hipStream_t s) {
  return launch_decode_mode(D, dtype, 1, q, k_pool, v_pool, page_table, seq_lens, sel_idx, sel_cnt, alpha,
                            tau_method, out, tau, weights_out, ws, ws_bytes, s);
}

hipError_t launch_entmax_full(const Dims &D, int dtype, const void *q, const void *k_pool, const void *v_pool,
                              const int32_t *page_table, const int32_t *seq_lens, double alpha, int tau_method,
                              float *out, double *tau, float *weights_out, void *ws, size_t ws_bytes,
                              hipStream_t s) {
  return launch_decode_mode(D, dtype, 2, q, k_pool, v_pool, page_table, seq_lens, nullptr, nullptr, alpha,
                            tau_method, out, tau, weights_out, ws, ws_bytes, s);
}

EKV_TRACE_DUMP(ekv_trace_dump_decode)
}  // namespace ekv
