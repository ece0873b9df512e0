// score.hip -- query-aware page scoring ([EntmaxKV s.2.A]).
//
// EntmaxKV s.2.A = section 2.A ("query-aware page scoring") of "Resumen Tecnico:
// EntmaxKV - Decodificacion Consciente del Soporte para Atencion Entmax",
// gist.science/es/paper/2605.21649: the bounding box (k_min, k_max) gives a
// deterministic upper bound on every score in the page, and the per-page key
// mean/variance give a Gaussian model of the page's scores.
//
// Per (b, h, p):  box = c sum_i max(q_i kmin_i, q_i kmax_i)
//                 mu  = c sum_i q_i mean_i,   var = c^2 sum_i q_i^2 var_i.
//
// The kernel is bound by the metadata stream (one record per page and KV head,
// rows kmin | kmax | mean | var of d elements each).  Design:
//  * a block scores two tiles of 64 logical pages of one (b, KV head g); the G
//    query heads of the group share every record read (GQA reuse);
//  * the four waves of the block split the record's work, lane = page: waves 0
//    and 1 each form the box of half of the G query heads from the k_min and
//    k_max rows (per coordinate, in index order, both exact products are added,
//    one of them with a zero coefficient, so the fp64 sum is the definition's
//    sum of max(q_i kmin_i, q_i kmax_i) added in the same order, bit for bit),
//    wave 2 forms mu from the mean row and wave 3 var from the variance row;
//  * tiles are fetched with coalesced 16-byte vector loads into registers (the
//    second tile while the first is scored), then written to LDS with
//    the 16-byte chunks of each record XOR-swizzled by the record index, so that
//    the lane-per-record reads of the compute hit distinct banks;
//  * the query-derived coefficients (q-, q+, q, q^2 in fp64, one table per
//    (b, g) row, laid out so that each wave reads one contiguous region in
//    coordinate order) are written once to a workspace table at the start and
//    read back through scalar loads, so the inner loop is fp64 FMAs on exact
//    products with a wave-uniform operand.  The table's
//    lines are pulled into the scalar cache with one batch of loads that overlaps
//    the tile fetch: otherwise the first tile's compute issues its coefficient
//    loads a few lines at a time, each a full L2 round trip behind the stream;
//  * the blocks that share a CU (on MI355X block i runs beside i + n_cu,
//    i + 2 n_cu, ...) are given consecutive tiles of the same row, so one
//    coefficient table serves the CU's scalar cache;
//  * outputs stay in registers until both tiles are scored, so that the vector
//    memory queue holds only loads while tiles are in flight (a store among them
//    would make every later wait drain the whole queue).
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace ekv {

constexpr int kTilePages = 64;      // one page per lane
static_assert(kTilePages == kSummaryTile, "one bracket summary entry per tile");
constexpr int kScoreThreads = 256;  // four waves: box (two), mean, variance
constexpr int kScoreTiles = 2;      // tiles per block
static_assert(kScoreTiles * kTilePages <= kScoreThreads, "one page id per thread in the prologue");

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Chunk;  // 16 bytes of one metadata row
template <>
struct Chunk<uint16_t> {
  static constexpr int kElems = 8;
  __device__ static void unpack(const uint4 &v, double *o) {
    o[0] = bf16lo(v.x); o[1] = bf16hi(v.x); o[2] = bf16lo(v.y); o[3] = bf16hi(v.y);
    o[4] = bf16lo(v.z); o[5] = bf16hi(v.z); o[6] = bf16lo(v.w); o[7] = bf16hi(v.w);
  }
};
template <>
struct Chunk<float> {
  static constexpr int kElems = 4;
  __device__ static void unpack(const uint4 &v, double *o) {
    o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
  }
};

// OCP FP8 E4M3 code -> fp64, exact: the code's exponent and mantissa bits set
// at the top of an fp64 give 2^(e - 1023) (1 + m/8) (a subnormal when e = 0,
// m/8 2^-1022); scaling by 2^1016 turns the bias into the format's 7.  The
// codes 0x7F / 0xFF are NaN.
__device__ __forceinline__ double e4m3_to_f64(unsigned c) {
  const unsigned hi = ((c & 0x7Fu) << 17) | ((c & 0x80u) << 24);
  const double v = __hiloint2double((int)hi, 0) * 0x1p1016;
  return (c & 0x7Fu) == 0x7Fu ? __builtin_nan("") : v;
}

// F8: compact records (bf16 k_min | k_max, then E4M3 mean | var: 6 DIM bytes)
template <typename T, int DIM, int G, bool F8>
struct ScoreCfg {
  static_assert(!F8 || sizeof(T) == 2, "compact records hold bf16 bounds");
  static constexpr int kE = Chunk<T>::kElems;          // elements per 16-byte chunk
  static constexpr int kRowChunks = DIM / kE;          // chunks per (box) metadata row
  static constexpr int kF8Chunks = DIM / 16;           // chunks per E4M3 row
  static constexpr int kRecBytes = F8 ? 6 * DIM : 4 * DIM * (int)sizeof(T);
  // a tile is staged in parts of the coordinates (every row's same range), 512
  // bytes of each record per part, so a part's tile is 32 KB and four blocks fit
  // a CU at every (d, dtype); the compact records stay whole
  static constexpr int kParts = F8 ? 1 : (kRecBytes > 512 ? kRecBytes / 512 : 1);
  static constexpr int kPartRec = kRecBytes / kParts;                  // bytes of a record per part
  static constexpr int kRowPartChunks = kRowChunks / kParts;           // chunks of a row per part
  static constexpr int kTileBytes = kTilePages * kPartRec;             // LDS stage: one part of a tile
  static constexpr int kLoads = kTileBytes / 16 / kScoreThreads;       // 16-byte loads per thread per part
  static constexpr int kLds = kTileBytes + kScoreTiles * (kTilePages + 1) * 4;
  static constexpr int kBlocksPerCu = (160 * 1024) / (kLds + 1024) >= 4 ? 4 : (160 * 1024) / (kLds + 1024);
  // coefficient table, doubles per (b, g) row: [box wave][i][j][q-, q+] (head
  // h = wave * kGH + j), then [i][h] of q (mean) and of q^2 (variance), so each
  // wave reads one contiguous region in coordinate order
  static constexpr int kGH = G > 1 ? G / 2 : 1;          // box heads per box wave
  static constexpr int kCoefRow = 4 * DIM * G;
  static constexpr int kWarmLines = DIM * G * 8 / 64;    // 64-byte lines of one wave's region (G > 1)
};

// Tile loads, part `part` of the coordinates: thread t fetches 16-byte chunks
// u*256 + t of the part's tile (chunk pos of a record's part is chunk c of row
// pos / kRowPartChunks, c = part * kRowPartChunks + pos % kRowPartChunks; a
// wave instruction covers runs of consecutive bytes); missing pages read
// record 0 and are masked later.
template <typename T, int DIM, int G, bool F8, int L>
__device__ __forceinline__ void score_load_tile(u32x4 (&r)[L], const char *mbase, const int *phys, int g, int hkv,
                                                int tid, int part) {
  using C = ScoreCfg<T, DIM, G, F8>;
#pragma unroll
  for (int u = 0; u < L; ++u) {
    const int off = (u * kScoreThreads + tid) * 16;
    const int rec = off / C::kPartRec, pos = (off % C::kPartRec) / 16;
    const int gpos = C::kParts == 1 ? pos
                                    : (pos / C::kRowPartChunks) * C::kRowChunks + part * C::kRowPartChunks +
                                          pos % C::kRowPartChunks;
    const int ph = max(phys[rec], 0);
    r[u] = *reinterpret_cast<const u32x4 *>(mbase + ((size_t)ph * hkv + g) * C::kRecBytes + gpos * 16);
  }
}
// ... and into LDS, chunk pos of record rec's part at slot pos ^ (rec & 7)
template <typename T, int DIM, int G, bool F8, int L>
__device__ __forceinline__ void score_stash_tile(const u32x4 (&r)[L], unsigned char *buf, int tid) {
  using C = ScoreCfg<T, DIM, G, F8>;
#pragma unroll
  for (int u = 0; u < L; ++u) {
    const int off = (u * kScoreThreads + tid) * 16;
    const int rec = off / C::kPartRec, pos = (off % C::kPartRec) / 16;
    *reinterpret_cast<u32x4 *>(buf + rec * C::kPartRec + ((pos ^ (rec & 7)) * 16)) = r[u];
  }
}

// Zeroes block bi's share of the n words at z (SUM variant: the Gaussian
// selector's counts and arrival counters, read by its next launches).
__device__ __forceinline__ void zero_share(const ScoreSummary &sm, int bi, int nb, int tid) {
  const long long per = (sm.nzero + nb - 1) / nb, z0 = (long long)bi * per;
  const long long z1 = z0 + per < sm.nzero ? z0 + per : sm.nzero;
  for (long long i = z0 + tid; i < z1; i += kScoreThreads) sm.zero[i] = 0u;
}

// SUM: also writes, per (query row, tile), the two maxima the Gaussian
// selector's bracket is made of (see the epilogue).
template <typename T, int DIM, int G, bool F8, bool SUM>
__global__ __launch_bounds__(kScoreThreads, (ScoreCfg<T, DIM, G, F8>::kBlocksPerCu)) void score_pages_kernel(
    Dims D, int tiles_per_row, int n_cu, const T *__restrict__ q, const T *__restrict__ meta,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ seq_lens, double *__restrict__ coef_w,
    const double *__restrict__ coef_r, float *__restrict__ box, float *__restrict__ mu,
    float *__restrict__ var, ScoreSummary sm) {
  using C = ScoreCfg<T, DIM, G, F8>;
  constexpr int kE = C::kE;
  constexpr int kGH = C::kGH;  // box heads of each of waves 0 and 1 (G = 1: wave 0 only)
  __shared__ __align__(16) unsigned char tile[C::kTileBytes];
  __shared__ int s_phys[kScoreTiles][kTilePages];
  __shared__ int s_np[kScoreTiles];
  __shared__ int s_zero;

  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // 0, 1 box; 2 mean; 3 variance
  const int n_tiles = D.B * D.Hkv * tiles_per_row;
  // blocks resident on one CU (i, i + n_cu, ...) take consecutive tile pairs
  const int nb = gridDim.x, bi = blockIdx.x;
  const int lb = (n_cu > 0 && nb % n_cu == 0) ? (bi % n_cu) * (nb / n_cu) + bi / n_cu : bi;
  const int t_begin = lb * kScoreTiles;
  const int t_end = min(n_tiles, t_begin + kScoreTiles);
  if (t_begin >= t_end) {
    if constexpr (SUM) zero_share(sm, bi, nb, tid);
    return;
  }
  const int nt = t_end - t_begin;
  const char *mbase = reinterpret_cast<const char *>(meta);
  const int row0 = t_begin / tiles_per_row, nrows = (t_end - 1) / tiles_per_row - row0 + 1;
  EKV_MARK(0, 0);

  // ---- prologue, one round trip: page ids (missing pages / bad ids -> -1) and q;
  // then the coefficient table of the block's rows, completed before any tile load
  // is issued (every block that scores row (b, g) stores the same bytes).
  {
    const int k = min(tid, nt * kTilePages - 1);
    const int t = t_begin + k / kTilePages;
    const int b = t / tiles_per_row / D.Hkv;
    const int p = min((t % tiles_per_row) * kTilePages + k % kTilePages, D.max_pages - 1);
    const int len = seq_lens[b];
    const int ph0 = page_table[(size_t)b * D.max_pages + p];
    // coefficient rows, one (b, g) at a time: entry tt = i G + h of row (b, g)
    // is built from q[b, g G + h, i]; the row's (b, g) is uniform
    {
      const int b0 = row0 / D.Hkv;
      int bb = b0, gg = row0 - b0 * D.Hkv;
#pragma unroll 1
      for (int rr = 0; rr < nrows; ++rr) {
        const T *qrow = q + ((size_t)bb * D.Hq + (size_t)gg * G) * DIM;
        double *cw = coef_w + (size_t)(row0 + rr) * C::kCoefRow;
#pragma unroll
        for (int tt = tid; tt < DIM * G; tt += kScoreThreads) {
          // entry tt = i G + h; box pair (q- for kmin, q+ for kmax) of head h
          // at box wave h / kGH, slot j = h % kGH
          const int i = tt / G, h = tt % G;
          const double qq = (double)load_f<T>(qrow, h * DIM + i);
          const int bw = G > 1 ? h / C::kGH : 0, j = G > 1 ? h % C::kGH : 0;
          double *pb = cw + (((size_t)bw * DIM + i) * C::kGH + j) * 2;
          pb[0] = qq < 0.0 ? qq : 0.0;
          pb[1] = qq >= 0.0 ? qq : 0.0;
          cw[2 * DIM * G + tt] = qq;
          cw[3 * DIM * G + tt] = qq * qq;
        }
        if (++gg == D.Hkv) { gg = 0; ++bb; }
      }
    }
    if (tid < nt * kTilePages) {
      const int lt = tid / kTilePages, r = tid % kTilePages;
      const int np = n_pages_of(len < 0 ? 0 : min(len, D.max_pages * D.P), D.P);
      const int pp = ((t_begin + lt) % tiles_per_row) * kTilePages + r;
      int ph = pp < np ? ph0 : -1;
      if (ph < 0 || ph >= D.num_phys) ph = -1;
      s_phys[lt][r] = ph;
      if (r == 0) s_np[lt] = np;
    }
    if (tid == 0) s_zero = 0;
  }
  // vmcnt(0): the table's stores have completed before its lines are loaded back
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
  lds_barrier();
  EKV_MARK(0, 1);

  // The table is read only after the barrier: the offset below is a zero the block
  // wrote to LDS before it, so no load of the table can be scheduled earlier.
  // (coef_r stays restrict-qualified, which lets the reads be scalar loads.)
  const int zoff = __builtin_amdgcn_readfirstlane(s_zero);
  // this wave's region of the coefficient table: its box heads' (q-, q+)
  // pairs, q (mean) or q^2 (variance)
  const size_t region = wave < 2 ? (size_t)wave * DIM * C::kGH * 2 : (size_t)wave * DIM * G;
  const double *cf0 = coef_r + zoff + (size_t)row0 * C::kCoefRow + region;
  // scalar-cache warm-up: one load per 64-byte line of this wave's coefficients,
  // all in flight together; consumed before the first tile is scored
  unsigned warm = 0;
  {
    const unsigned *cl = reinterpret_cast<const unsigned *>(cf0);
#pragma unroll
    for (int i = 0; i < C::kWarmLines; ++i) warm ^= cl[i * 16];
    if (G == 1 && wave == 0) {  // the lone box wave's region holds two doubles per coordinate
#pragma unroll
      for (int i = 0; i < C::kWarmLines; ++i) warm ^= cl[(C::kWarmLines + i) * 16];
    }
  }
  // two register buffers: step st + 1 (a part of a tile) is requested once step
  // st is in LDS (with more in flight from the start the per-tile latency grows
  // with the deeper memory queue and the first tile arrives later, measured on
  // cold HBM)
  constexpr int NP = C::kParts;
  u32x4 ring[2][C::kLoads];
  // tile loads are issued at raised wave priority (measured: 0.1-0.6 us per launch
  // faster; the whole prologue at raised priority was slower)
  __builtin_amdgcn_s_setprio(3);
  score_load_tile<T, DIM, G, F8>(ring[0], mbase, s_phys[0], row0 % D.Hkv, D.Hkv, tid, 0);
  __builtin_amdgcn_s_setprio(0);

  const double c = D.scale, c2 = D.scale * D.scale;
  const unsigned char *rec = tile + lane * C::kPartRec;
  const int sw = lane & 7;
  float outv[kScoreTiles][G];
#pragma unroll
  for (int lt = 0; lt < kScoreTiles; ++lt)
#pragma unroll
    for (int h = 0; h < G; ++h) outv[lt][h] = 0.f;

#pragma unroll
  for (int lt = 0; lt < kScoreTiles; ++lt) {
    if (lt < nt) {
      // ---- lane = page.  Box waves: acc[j] = sum_i (q-_i kmin_i + q+_i kmax_i)
      // for head h0 + j, coordinate by coordinate; mean / variance waves:
      // acc[h] = sum_i coef[i][h] * row_i (q for the mean row, q^2 for the variance row).
      // The parts come in coordinate order, so the sums run over i in index order.
      const int row = (t_begin + lt) / tiles_per_row;
      const double *cf = cf0 + (size_t)(row - row0) * C::kCoefRow;
      const bool ok = s_phys[lt][lane] >= 0;
      double acc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = 0.0;
#pragma unroll
      for (int part = 0; part < NP; ++part) {
        const int st = lt * NP + part;
        if (st > 0) lds_barrier();  // the previous step is fully read
        score_stash_tile<T, DIM, G, F8>(ring[st & 1], tile, tid);
        asm volatile("" ::: "memory");
        if (st + 1 < nt * NP) {
          const int nl = (st + 1) / NP, np_ = (st + 1) % NP;
          __builtin_amdgcn_s_setprio(3);  // the loads issue ahead of other waves' FMA stream
          score_load_tile<T, DIM, G, F8>(ring[(st + 1) & 1], mbase, s_phys[nl],
                                         ((t_begin + nl) / tiles_per_row) % D.Hkv, D.Hkv, tid, np_);
          __builtin_amdgcn_s_setprio(0);
        }
        lds_barrier();
        if (st == 0) asm volatile("" ::"s"(warm));
        if (st == 0) EKV_MARK(0, 2);
        const int i0 = part * C::kRowPartChunks * kE;  // first coordinate of the part
        if (wave < 2) {
          if (G > 1 || wave == 0) {  // wave-uniform
#pragma unroll 2
            for (int ch = 0; ch < C::kRowPartChunks; ++ch) {
              double xn[kE], xp[kE];
              Chunk<T>::unpack(*reinterpret_cast<const uint4 *>(rec + (ch ^ sw) * 16), xn);
              Chunk<T>::unpack(*reinterpret_cast<const uint4 *>(rec + ((C::kRowPartChunks + ch) ^ sw) * 16), xp);
#pragma unroll
              for (int e = 0; e < kE; ++e) {
                const double *ci = cf + (size_t)(i0 + ch * kE + e) * kGH * 2;
#pragma unroll
                for (int j = 0; j < kGH; ++j) {
                  // exact products (bf16 x bf16 in 16 bits, f32 x f32 in 48): fused == separate
                  acc[j] = __builtin_fma(ci[2 * j], xn[e], acc[j]);
                  acc[j] = __builtin_fma(ci[2 * j + 1], xp[e], acc[j]);
                }
              }
            }
          }
        } else if (!F8) {
#pragma unroll 2
          for (int ch = 0; ch < C::kRowPartChunks; ++ch) {
            double x[kE];
            Chunk<T>::unpack(*reinterpret_cast<const uint4 *>(rec + ((wave * C::kRowPartChunks + ch) ^ sw) * 16), x);
#pragma unroll
            for (int e = 0; e < kE; ++e) {
              const double *ci = cf + (size_t)(i0 + ch * kE + e) * G;
#pragma unroll
              for (int h = 0; h < G; ++h) {
                if constexpr (sizeof(T) == 2)
                  acc[h] = __builtin_fma(ci[h], x[e], acc[h]);  // exact product: fused == separate
                else
                  acc[h] = acc[h] + ci[h] * x[e];               // fp32 keys: q^2 var rounds, as defined
              }
            }
          }
        } else {
          // E4M3 mean / variance rows: 16 elements per chunk; q (bf16) times an
          // E4M3 value has 12 significant bits, q^2 times one 20: exact in fp64
          const int base = 2 * C::kRowChunks + (wave - 2) * C::kF8Chunks;
#pragma unroll 2
          for (int ch = 0; ch < C::kF8Chunks; ++ch) {
            const uint4 v = *reinterpret_cast<const uint4 *>(rec + ((base + ch) ^ sw) * 16);
            const unsigned w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const double xe = e4m3_to_f64((w4[e >> 2] >> (8 * (e & 3))) & 0xFFu);
              const double *ci = cf + (size_t)(ch * 16 + e) * G;
#pragma unroll
              for (int h = 0; h < G; ++h) acc[h] = __builtin_fma(ci[h], xe, acc[h]);
            }
          }
        }
      }
      if (wave < 2) {
        if (G > 1 || wave == 0) {
#pragma unroll
          for (int j = 0; j < kGH; ++j) outv[lt][j] = ok ? __double2float_ru(c * acc[j]) : NAN;
        }
      } else {
        const double sc = wave == 2 ? c : c2;
#pragma unroll
        for (int h = 0; h < G; ++h) outv[lt][h] = ok ? (float)(sc * acc[h]) : NAN;
      }
    }
  }
  EKV_MARK(0, 3);

  if constexpr (SUM) {
    // The Gaussian selector's bracket from the values as stored (fp32), per
    // (query row, tile): the largest mean over the tile's valid full pages and
    // the largest top quadrature point mu + sqrt2 sigma x_16 over its valid
    // pages (valid: box, mu and var finite).  Scaling by alpha - 1 > 0 and
    // subtracting a constant are monotone in fp64, so the selector's bracket
    // from these maxima has the bits of its own per-page maxima.
    // Every wave hands its values to LDS; then wave w takes heads w, w + 4, ...
    __shared__ float s_sb[kScoreTiles][G][kTilePages], s_sm[kScoreTiles][G][kTilePages],
        s_sv[kScoreTiles][G][kTilePages];
#pragma unroll
    for (int lt = 0; lt < kScoreTiles; ++lt) {
      if (wave < 2) {
        if (G > 1 || wave == 0) {
#pragma unroll
          for (int j = 0; j < kGH; ++j) s_sb[lt][G == 1 ? 0 : wave * kGH + j][lane] = outv[lt][j];
        }
      } else {
#pragma unroll
        for (int h = 0; h < G; ++h) (wave == 2 ? s_sm : s_sv)[lt][h][lane] = outv[lt][h];
      }
    }
    lds_barrier();
#pragma unroll 1
    for (int h = wave; h < G; h += 4) {
#pragma unroll
      for (int lt = 0; lt < kScoreTiles; ++lt) {
        if (lt < nt) {
          const int t = t_begin + lt;
          const int row = t / tiles_per_row;
          const int b = row / D.Hkv, g = row - b * D.Hkv, tin = t - row * tiles_per_row;
          const int p = tin * kTilePages + lane;
          const long long L = seq_len_clamped(seq_lens, b, D);
          const float m = s_sm[lt][h][lane], v2 = s_sv[lt][h][lane], bx = s_sb[lt][h][lane];
          const bool valid = p < s_np[lt] && isfinite(bx) && isfinite(m) && isfinite(v2);
          const double md = (double)m;
          double m1 = valid && (long long)(p + 1) * D.P <= L ? md : -INFINITY;
          double tp = valid ? md + 1.4142135623730951 * sqrt(v2 > 0.0f ? (double)v2 : 0.0) * sm.x_top : -INFINITY;
          m1 = wave_max(m1);
          tp = wave_max(tp);
          if (lane == 0) {
            double *o = sm.summ + (((size_t)b * D.Hq + g * G + h) * tiles_per_row + tin) * 2;
            o[0] = m1;
            o[1] = tp;
          }
        }
      }
    }
  }

  // ---- outputs: lane = page, 64 consecutive floats per (kind, head) and tile
#pragma unroll
  for (int lt = 0; lt < kScoreTiles; ++lt) {
    if (lt < nt) {
      const int t = t_begin + lt;
      const int row = t / tiles_per_row;
      const int b = row / D.Hkv, g = row - b * D.Hkv;
      const int p = (t - row * tiles_per_row) * kTilePages + lane;
      if (p < s_np[lt]) {
        if (wave < 2) {
          if (G > 1 || wave == 0) {
#pragma unroll
            for (int j = 0; j < kGH; ++j) {
              const int h = G == 1 ? 0 : wave * kGH + j;
              box[((size_t)b * D.Hq + g * G + h) * D.max_pages + p] = outv[lt][j];
            }
          }
        } else {
          float *dst = wave == 2 ? mu : var;
#pragma unroll
          for (int h = 0; h < G; ++h) dst[((size_t)b * D.Hq + g * G + h) * D.max_pages + p] = outv[lt][h];
        }
      }
    }
  }
  if constexpr (SUM) zero_share(sm, bi, nb, tid);
  EKV_MARK(0, 4);
}

size_t score_ws_bytes(const Dims &D) {
  Carve cv(nullptr);
  cv.take<double>((size_t)D.B * D.Hkv * 4 * D.d * D.G);
  return cv.bytes();
}

static int device_cu_count() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = -1;
    cached[dev] = n;
  }
  return cached[dev] > 0 ? cached[dev] : 0;
}

template <typename T, int DIM, int G, bool F8, bool SUM>
static hipError_t launch_score_t(const Dims &D, const void *q, const void *meta,
                                 const int32_t *page_table, const int32_t *seq_lens, float *box,
                                 float *mu, float *var, void *ws, const ScoreSummary &sm, hipStream_t s) {
  Carve cv(ws);
  double *coef = cv.take<double>((size_t)D.B * D.Hkv * 4 * D.d * D.G);
  const int tiles_per_row = (D.max_pages + kTilePages - 1) / kTilePages;
  const long long n_tiles = (long long)D.B * D.Hkv * tiles_per_row;
  const long long grid = (n_tiles + kScoreTiles - 1) / kScoreTiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((score_pages_kernel<T, DIM, G, F8, SUM>), dim3((unsigned)grid), dim3(kScoreThreads), 0, s, D,
                     tiles_per_row, device_cu_count(), (const T *)q, (const T *)meta, page_table, seq_lens, coef,
                     (const double *)coef, box, mu, var, sm);
  return hipGetLastError();
}

template <typename T, int DIM, bool F8, bool SUM = false>
static hipError_t launch_score_d(const Dims &D, const void *q, const void *meta,
                                 const int32_t *pt, const int32_t *sl, float *box, float *mu,
                                 float *var, void *ws, hipStream_t s, const ScoreSummary &sm = ScoreSummary{}) {
  switch (D.G) {
    case 1: return launch_score_t<T, DIM, 1, F8, SUM>(D, q, meta, pt, sl, box, mu, var, ws, sm, s);
    case 2: return launch_score_t<T, DIM, 2, F8, SUM>(D, q, meta, pt, sl, box, mu, var, ws, sm, s);
    case 4: return launch_score_t<T, DIM, 4, F8, SUM>(D, q, meta, pt, sl, box, mu, var, ws, sm, s);
    case 8: return launch_score_t<T, DIM, 8, F8, SUM>(D, q, meta, pt, sl, box, mu, var, ws, sm, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_score(const Dims &D, int dtype, bool f8, const void *q, const void *meta,
                        const int32_t *page_table, const int32_t *seq_lens, float *box, float *mu,
                        float *var, void *ws, hipStream_t s) {
  if (dtype == ENTMAXKV_BF16 && f8) {
    if (D.d == 64) return launch_score_d<uint16_t, 64, true>(D, q, meta, page_table, seq_lens, box, mu, var, ws, s);
    return launch_score_d<uint16_t, 128, true>(D, q, meta, page_table, seq_lens, box, mu, var, ws, s);
  }
  if (f8) return hipErrorInvalidValue;
  if (dtype == ENTMAXKV_BF16) {
    if (D.d == 64) return launch_score_d<uint16_t, 64, false>(D, q, meta, page_table, seq_lens, box, mu, var, ws, s);
    return launch_score_d<uint16_t, 128, false>(D, q, meta, page_table, seq_lens, box, mu, var, ws, s);
  }
  if (D.d == 64) return launch_score_d<float, 64, false>(D, q, meta, page_table, seq_lens, box, mu, var, ws, s);
  return launch_score_d<float, 128, false>(D, q, meta, page_table, seq_lens, box, mu, var, ws, s);
}

hipError_t launch_score_summary(const Dims &D, int dtype, const void *q, const void *meta,
                                const int32_t *page_table, const int32_t *seq_lens, float *box, float *mu,
                                float *var, void *ws, const ScoreSummary &sm, hipStream_t s) {
  if (dtype == ENTMAXKV_BF16) {
    if (D.d == 64)
      return launch_score_d<uint16_t, 64, false, true>(D, q, meta, page_table, seq_lens, box, mu, var, ws, s, sm);
    return launch_score_d<uint16_t, 128, false, true>(D, q, meta, page_table, seq_lens, box, mu, var, ws, s, sm);
  }
  if (D.d == 64) return launch_score_d<float, 64, false, true>(D, q, meta, page_table, seq_lens, box, mu, var, ws, s, sm);
  return launch_score_d<float, 128, false, true>(D, q, meta, page_table, seq_lens, box, mu, var, ws, s, sm);
}

size_t score_summary_doubles(const Dims &D) {
  return (size_t)D.B * D.Hq * ((D.max_pages + kTilePages - 1) / kTilePages) * 2;
}

// ---------------------------------------------------- allocation-free variant
// score_pages_noalloc takes the coefficient table from this file-scope device
// array instead of a caller workspace.  Each GPU the library runs on holds its
// own copy until the process ends.  The kernel writes every table row it reads
// before reading it, so nothing in it has to start at zero; two calls that
// overlap on one GPU share the array and race.
constexpr size_t kScoreScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) unsigned char scratch[kScoreScratchBytes];

size_t score_scratch_bytes() { return kScoreScratchBytes; }

// Device address of `scratch` on the current device, looked up once per device
// (the host-side name of the array is not a device address).
static hipError_t scratch_address(void **out) {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static void *addr[kMaxDev];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_score_noalloc(const Dims &D, int dtype, const void *q, const void *meta,
                                const int32_t *page_table, const int32_t *seq_lens, float *box, float *mu,
                                float *var, hipStream_t s) {
  if (score_ws_bytes(D) > kScoreScratchBytes) return hipErrorInvalidValue;  // checked by the caller first
  void *ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  return launch_score(D, dtype, false, q, meta, page_table, seq_lens, box, mu, var, ws, s);
}

EKV_TRACE_DUMP(ekv_trace_dump_score)
}  // namespace ekv
