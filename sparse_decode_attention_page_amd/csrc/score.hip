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
// 4*d elements).  Design:
//  * work unit = one (b, KV head g) and a tile of 64 logical pages; the G query
//    heads of the group share every record read (GQA reuse);
//  * persistent blocks walk a contiguous run of tiles with NBUF tile buffers in
//    LDS: tiles t+1 .. t+NBUF-1 stream in with global_load_lds (16 bytes per
//    lane, straight to LDS, no staging registers) while tile t is computed;
//  * inside a record the 16-byte chunks are XOR-swizzled by the record index,
//    so the lane-per-page reads of one chunk hit distinct LDS banks; the global
//    side stays fully coalesced (a wave fetches whole records, permuted);
//  * each wave owns a quarter of the coordinates, each lane one page; the
//    query-derived coefficients (q+, q-, q, q^2 in fp64) are wave-uniform, written
//    once per (b, g) to a workspace table and read back through scalar loads, so
//    the inner loop is four fp64 FMAs per (coordinate, head) on exact products;
//  * the four coordinate quarters are combined in a fixed order.
#include "common.hpp"
#include "launch.hpp"

namespace ekv {

constexpr int kTilePages = 64;
constexpr int kScoreThreads = 256;
constexpr int kMaxTilesPerBlock = 16;
constexpr size_t kScoreLds = 160 * 1024;

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

template <typename T, int DIM, int G>
struct ScoreCfg {
  static constexpr int kRecBytes = 4 * DIM * (int)sizeof(T);
  static constexpr int kRecChunks = kRecBytes / 16;
  static constexpr int kTileBytes = kTilePages * kRecBytes;
  static constexpr int kRedBytes = 4 * 3 * G * kWave * 8;
  static constexpr bool kRedInTile = kRedBytes <= kTileBytes;
  // One tile buffer per block: LDS-DMA throughput grows with the number of
  // waves issuing it, so LDS goes to more resident blocks per CU rather than
  // to deeper per-block prefetch; the blocks of a CU overlap each other's
  // loads and compute.
  static constexpr int kNBuf = 1;
  static constexpr size_t kLds = (size_t)kNBuf * kTileBytes + (kRedInTile ? 0 : kRedBytes);
  static constexpr int kBlocksPerCu = (int)(kScoreLds / (kLds + 8 * 1024)) < 1 ? 1 : (int)(kScoreLds / (kLds + 8 * 1024));
  static constexpr int kLoadsPerWave = kTileBytes / 1024 / 4;  // 1 KB per wave instruction
  static_assert(kLds <= kScoreLds, "tile does not fit in LDS");
  static_assert(kTileBytes % 4096 == 0, "tile split across 4 waves");
};

__device__ __forceinline__ void wait_vmcnt(int n) {
  // s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
  // vmcnt[3:0] | expcnt[6:4]=7 | lgkmcnt[11:8]=15 | vmcnt[5:4] << 14)
  switch (n) {
#define EKV_W(k) case k: __builtin_amdgcn_s_waitcnt(((k) & 15) | (7 << 4) | (15 << 8) | (((k) >> 4) << 14)); break;
    EKV_W(0) EKV_W(1) EKV_W(2) EKV_W(3) EKV_W(4) EKV_W(5) EKV_W(6) EKV_W(7) EKV_W(8) EKV_W(9) EKV_W(10)
    EKV_W(11) EKV_W(12) EKV_W(13) EKV_W(14) EKV_W(15) EKV_W(16) EKV_W(17) EKV_W(18) EKV_W(19) EKV_W(20)
    EKV_W(21) EKV_W(22) EKV_W(23) EKV_W(24) EKV_W(25) EKV_W(26) EKV_W(27) EKV_W(28) EKV_W(29) EKV_W(30)
    EKV_W(31) EKV_W(32) EKV_W(33) EKV_W(34) EKV_W(35) EKV_W(36) EKV_W(37) EKV_W(38) EKV_W(39) EKV_W(40)
    EKV_W(41) EKV_W(42) EKV_W(43) EKV_W(44) EKV_W(45) EKV_W(46) EKV_W(47) EKV_W(48) EKV_W(49) EKV_W(50)
    EKV_W(51) EKV_W(52) EKV_W(53) EKV_W(54) EKV_W(55) EKV_W(56) EKV_W(57) EKV_W(58) EKV_W(59) EKV_W(60)
    EKV_W(61) EKV_W(62) EKV_W(63)
#undef EKV_W
    default: __builtin_amdgcn_s_waitcnt(0); break;
  }
}

template <typename T, int DIM, int G>
__global__ __launch_bounds__(kScoreThreads) void score_pages_kernel(
    Dims D, int tiles_per_row, int tiles_per_block, const T *__restrict__ q, const T *__restrict__ meta,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ seq_lens, double *__restrict__ coef_w,
    const double *__restrict__ coef_r, float *__restrict__ box, float *__restrict__ mu,
    float *__restrict__ var) {
  using C = ScoreCfg<T, DIM, G>;
  constexpr int kE = Chunk<T>::kElems;  // elements per 16-byte chunk
  constexpr int kRowChunks = DIM / kE;   // chunks per metadata row
  constexpr int kQChunks = DIM / 4 / kE; // chunks per coordinate quarter

  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_phys[kMaxTilesPerBlock][kTilePages];
  __shared__ int s_np[kMaxTilesPerBlock];

  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n_tiles = D.B * D.Hkv * tiles_per_row;
  const int t_begin = blockIdx.x * tiles_per_block;
  const int t_end = min(n_tiles, t_begin + tiles_per_block);
  if (t_begin >= t_end) return;
  const int nt = t_end - t_begin;
  const char *mbase = reinterpret_cast<const char *>(meta);
  EKV_MARK(0, 0);

  // ---- prologue, one round trip: the page ids of every tile of the block
  // (missing pages / bad ids -> -1) and the coefficient table (q+, q-, q, q^2
  // in fp64) of every (b, g) row the block touches.  Every block that scores
  // (b, g) stores the same bytes into the same slot; the tile loop reads the
  // table back through scalar loads once the stores have completed.
  constexpr int kPtPer = kMaxTilesPerBlock * kTilePages / kScoreThreads;
  int pt_ph[kPtPer], pt_len[kPtPer];
#pragma unroll
  for (int u = 0; u < kPtPer; ++u) {
    const int k = min(u * kScoreThreads + tid, nt * kTilePages - 1);
    const int t = t_begin + k / kTilePages;
    const int b = t / tiles_per_row / D.Hkv;
    const int p = min((t % tiles_per_row) * kTilePages + k % kTilePages, D.max_pages - 1);
    pt_len[u] = seq_lens[b];
    pt_ph[u] = page_table[(size_t)b * D.max_pages + p];
  }
  {
    const int row0 = t_begin / tiles_per_row, nrows = (t_end - 1) / tiles_per_row - row0 + 1;
    const int n_coef = nrows * DIM * G;
#pragma unroll 1
    for (int k0 = 0; k0 < n_coef; k0 += 4 * kScoreThreads) {
      double qv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int k = min(k0 + u * kScoreThreads + tid, n_coef - 1);
        const int row = row0 + k / (DIM * G), tt = k % (DIM * G);
        const int b = row / D.Hkv, g = row % D.Hkv;
        qv[u] = (double)load_f<T>(q, ((size_t)b * D.Hq + g * G + tt % G) * DIM + tt / G);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int k = k0 + u * kScoreThreads + tid;
        if (k < n_coef) {
          double *c4 = coef_w + ((size_t)(row0 + k / (DIM * G)) * DIM * G + k % (DIM * G)) * 4;
          c4[0] = qv[u] >= 0.0 ? qv[u] : 0.0;
          c4[1] = qv[u] < 0.0 ? qv[u] : 0.0;
          c4[2] = qv[u];
          c4[3] = qv[u] * qv[u];
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kPtPer; ++u) {
    const int k = u * kScoreThreads + tid;
    if (k < nt * kTilePages) {
      const int lt = k / kTilePages, r = k % kTilePages;
      const int t = t_begin + lt;
      const int np = n_pages_of(pt_len[u] < 0 ? 0 : min(pt_len[u], D.max_pages * D.P), D.P);
      const int p = (t % tiles_per_row) * kTilePages + r;
      int ph = p < np ? pt_ph[u] : -1;
      if (ph < 0 || ph >= D.num_phys) ph = -1;
      s_phys[lt][r] = ph;
      if (r == 0) s_np[lt] = np;
    }
  }
  // page ids visible to the block; the coefficient stores are older than
  // every tile load, so the per-tile vmcnt wait plus the barrier that follows
  // it also cover them before the first scalar load of the table
  lds_barrier();
  EKV_MARK(0, 1);

  // ---- tile loads: wave w fetches LDS bytes [w*T/4, (w+1)*T/4) of the tile
  // buffer; lane l of instruction u lands at +16 l, which holds chunk
  // (pos ^ (rec & 7)) of record rec.
  auto issue_tile = [&](int lt) {
    const int t = t_begin + lt;
    const int g = (t / tiles_per_row) % D.Hkv;
    unsigned char *buf = smem + (size_t)(lt % C::kNBuf) * C::kTileBytes;
#pragma unroll
    for (int u = 0; u < C::kLoadsPerWave; ++u) {
      const int off = (wave * C::kLoadsPerWave + u) * 1024 + lane * 16;
      const int rec = off / C::kRecBytes, pos = (off % C::kRecBytes) / 16;
      const int chunk = pos ^ (rec & 7);
      const int ph = max(s_phys[lt][rec], 0);  // missing pages read record 0 and are masked later
      const char *src = mbase + ((size_t)ph * D.Hkv + g) * C::kRecBytes + (size_t)chunk * 16;
      __builtin_amdgcn_global_load_lds((const void *)src,
                                       (__attribute__((address_space(3))) void *)(buf + (wave * C::kLoadsPerWave + u) * 1024),
                                       16, 0, 0);
    }
  };
  for (int lt = 0; lt < C::kNBuf - 1 && lt < nt; ++lt) issue_tile(lt);  // tiles 0 .. NBUF-2
  EKV_MARK(0, 2);

  double *red = reinterpret_cast<double *>(C::kRedInTile ? smem : smem + (size_t)C::kNBuf * C::kTileBytes);
  for (int lt = 0; lt < nt; ++lt) {
    const int t = t_begin + lt;
    const int row = t / tiles_per_row, pt = t % tiles_per_row;
    const int b = row / D.Hkv, g = row % D.Hkv;
    const int p0 = pt * kTilePages;
    const int np = s_np[lt];
    unsigned char *buf = smem + (size_t)(lt % C::kNBuf) * C::kTileBytes;
    // ---- prefetch: tile lt+NBUF-1 goes into the buffer freed by tile lt-1
    // (with a single buffer this is tile lt itself)
    if (lt + C::kNBuf - 1 < nt) issue_tile(lt + C::kNBuf - 1);

    // ---- tile lt is resident once this wave's loads for it completed
    const int ahead = min(C::kNBuf - 1, nt - 1 - lt);  // tiles issued after lt
    wait_vmcnt(ahead * C::kLoadsPerWave);  // loads return in order: this covers all of tile lt
    lds_barrier();

    // ---- compute: wave = coordinate quarter, lane = page
    if (lt == 0) EKV_MARK(0, 3);
    double acc_b[G], acc_m[G], acc_v[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc_b[h] = acc_m[h] = acc_v[h] = 0.0;
    const double *cf = coef_r + (size_t)row * DIM * G * 4;
    const unsigned char *rec = buf + lane * C::kRecBytes;
    const int sw = lane & 7;
#pragma unroll 1
    for (int qc = 0; qc < kQChunks; ++qc) {
      const int chunk = wave * kQChunks + qc;  // chunk index within a row
      double kmin[kE], kmax[kE], kmean[kE], kvar[kE];
      Chunk<T>::unpack(*reinterpret_cast<const uint4 *>(rec + ((0 * kRowChunks + chunk) ^ sw) * 16), kmin);
      Chunk<T>::unpack(*reinterpret_cast<const uint4 *>(rec + ((1 * kRowChunks + chunk) ^ sw) * 16), kmax);
      Chunk<T>::unpack(*reinterpret_cast<const uint4 *>(rec + ((2 * kRowChunks + chunk) ^ sw) * 16), kmean);
      Chunk<T>::unpack(*reinterpret_cast<const uint4 *>(rec + ((3 * kRowChunks + chunk) ^ sw) * 16), kvar);
#pragma unroll
      for (int e = 0; e < kE; ++e) {
        const int i = chunk * kE + e;
        const double *ci = cf + (size_t)i * G * 4;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const double cpos = ci[h * 4 + 0], cneg = ci[h * 4 + 1], cq = ci[h * 4 + 2], cqq = ci[h * 4 + 3];
          acc_b[h] = __builtin_fma(cpos, kmax[e], acc_b[h]);
          acc_b[h] = __builtin_fma(cneg, kmin[e], acc_b[h]);
          acc_m[h] = __builtin_fma(cq, kmean[e], acc_m[h]);
          if constexpr (sizeof(T) == 2)
            acc_v[h] = __builtin_fma(cqq, kvar[e], acc_v[h]);  // exact product: fused == separate
          else
            acc_v[h] = acc_v[h] + cqq * kvar[e];               // fp32 keys: round the product first
        }
      }
    }
    // ---- combine the four coordinate quarters in a fixed order
    double *rd = C::kRedInTile ? reinterpret_cast<double *>(buf) : red;
    if (C::kRedInTile) lds_barrier();  // every wave is done reading the tile
#pragma unroll
    for (int h = 0; h < G; ++h) {
      rd[(wave * 3 * G + 0 * G + h) * kWave + lane] = acc_b[h];
      rd[(wave * 3 * G + 1 * G + h) * kWave + lane] = acc_m[h];
      rd[(wave * 3 * G + 2 * G + h) * kWave + lane] = acc_v[h];
    }
    lds_barrier();
    const double c = D.scale, c2 = D.scale * D.scale;
    for (int idx = tid; idx < 3 * G * kWave; idx += kScoreThreads) {
      const int k = idx / kWave, r = idx % kWave;
      const int p = p0 + r;
      if (p >= np) continue;
      double sacc = rd[(0 * 3 * G + k) * kWave + r];
      sacc += rd[(1 * 3 * G + k) * kWave + r];
      sacc += rd[(2 * 3 * G + k) * kWave + r];
      sacc += rd[(3 * 3 * G + k) * kWave + r];
      const int kind = k / G, h = g * G + (k % G);
      const size_t o = ((size_t)b * D.Hq + h) * D.max_pages + p;
      const bool ok = s_phys[lt][r] >= 0;
      if (kind == 0) box[o] = ok ? __double2float_ru(c * sacc) : NAN;
      else if (kind == 1) mu[o] = ok ? (float)(c * sacc) : NAN;
      else var[o] = ok ? (float)(c2 * sacc) : NAN;
    }
    lds_barrier();  // buffer lt % NBUF (and red) may be refilled from here on
  }
  EKV_MARK(0, 4);
}

size_t score_ws_bytes(const Dims &D) {
  Carve cv(nullptr);
  cv.take<double>((size_t)D.B * D.Hkv * D.d * D.G * 4);
  return cv.bytes();
}

template <typename T, int DIM, int G>
static hipError_t launch_score_t(const Dims &D, const void *q, const void *meta,
                                 const int32_t *page_table, const int32_t *seq_lens, float *box,
                                 float *mu, float *var, void *ws, hipStream_t s) {
  using C = ScoreCfg<T, DIM, G>;
  Carve cv(ws);
  double *coef = cv.take<double>((size_t)D.B * D.Hkv * D.d * D.G * 4);
  // persistent blocks (kBlocksPerCu per CU), each walking a contiguous run of tiles
  const int tiles_per_row = (D.max_pages + kTilePages - 1) / kTilePages;
  const int n_tiles = D.B * D.Hkv * tiles_per_row;
  const int slots = 256 * C::kBlocksPerCu;
  int tiles_per_block = (n_tiles + slots - 1) / slots;
  if (tiles_per_block > kMaxTilesPerBlock) tiles_per_block = kMaxTilesPerBlock;
  const int grid = (n_tiles + tiles_per_block - 1) / tiles_per_block;
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute((const void *)score_pages_kernel<T, DIM, G>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)C::kLds);
    attr_set = true;
  }
  hipLaunchKernelGGL((score_pages_kernel<T, DIM, G>), dim3(grid), dim3(kScoreThreads), C::kLds, s, D,
                     tiles_per_row, tiles_per_block, (const T *)q, (const T *)meta, page_table, seq_lens, coef,
                     (const double *)coef, box, mu, var);
  return hipGetLastError();
}

template <typename T, int DIM>
static hipError_t launch_score_d(const Dims &D, const void *q, const void *meta,
                                 const int32_t *pt, const int32_t *sl, float *box, float *mu,
                                 float *var, void *ws, hipStream_t s) {
  switch (D.G) {
    case 1: return launch_score_t<T, DIM, 1>(D, q, meta, pt, sl, box, mu, var, ws, s);
    case 2: return launch_score_t<T, DIM, 2>(D, q, meta, pt, sl, box, mu, var, ws, s);
    case 4: return launch_score_t<T, DIM, 4>(D, q, meta, pt, sl, box, mu, var, ws, s);
    case 8: return launch_score_t<T, DIM, 8>(D, q, meta, pt, sl, box, mu, var, ws, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_score(const Dims &D, int dtype, const void *q, const void *meta,
                        const int32_t *page_table, const int32_t *seq_lens, float *box, float *mu,
                        float *var, void *ws, hipStream_t s) {
  if (dtype == ENTMAXKV_BF16) {
    if (D.d == 64) return launch_score_d<uint16_t, 64>(D, q, meta, page_table, seq_lens, box, mu, var, ws, s);
    return launch_score_d<uint16_t, 128>(D, q, meta, page_table, seq_lens, box, mu, var, ws, s);
  }
  if (D.d == 64) return launch_score_d<float, 64>(D, q, meta, page_table, seq_lens, box, mu, var, ws, s);
  return launch_score_d<float, 128>(D, q, meta, page_table, seq_lens, box, mu, var, ws, s);
}

EKV_TRACE_DUMP(ekv_trace_dump_score)
}  // namespace ekv
