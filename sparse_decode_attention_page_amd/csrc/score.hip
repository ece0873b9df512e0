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
//  * one block = one (b, KV head g) and a tile of 64 logical pages; the G query
//    heads of the group share every record read (GQA reuse);
//  * the tile's records are fetched with coalesced 16-byte loads into LDS,
//    padded by 16 bytes per record so that lane-per-page reads are conflict free;
//  * each wave then owns a quarter of the coordinates and each lane one page;
//    the query-derived coefficients (q+, q-, q, q^2 in fp64) are wave-uniform
//    and come from a small table through scalar loads, so the inner loop is
//    four fp64 FMAs per (coordinate, head) on exact products;
//  * the four coordinate quarters are combined in a fixed order.
#include "common.hpp"
#include "launch.hpp"

namespace ekv {

constexpr int kTilePages = 64;
constexpr int kScoreThreads = 256;

// coef[((b*Hkv + g)*d + i)*G + hh][4] = {max(q,0), min(q,0), q, q*q}, q = q[b][g*G+hh][i]
template <typename T>
__global__ void score_coef_kernel(Dims D, const T *__restrict__ q, double *__restrict__ coef) {
  const int bg = blockIdx.x;  // b*Hkv + g
  const int b = bg / D.Hkv, g = bg % D.Hkv;
  for (int t = threadIdx.x; t < D.d * D.G; t += blockDim.x) {
    const int i = t / D.G, hh = t % D.G;
    const double qv = (double)load_f<T>(q, ((size_t)b * D.Hq + g * D.G + hh) * D.d + i);
    double *c = coef + (((size_t)bg * D.d + i) * D.G + hh) * 4;
    c[0] = qv >= 0.0 ? qv : 0.0;
    c[1] = qv < 0.0 ? qv : 0.0;
    c[2] = qv;
    c[3] = qv * qv;
  }
}

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
__global__ __launch_bounds__(kScoreThreads) void score_pages_kernel(
    Dims D, const T *__restrict__ meta, const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ seq_lens, const double *__restrict__ coef, float *__restrict__ box,
    float *__restrict__ mu, float *__restrict__ var) {
  constexpr int kRecBytes = 4 * DIM * (int)sizeof(T);
  constexpr int kStride = kRecBytes + 16;
  constexpr int kRecChunks = kRecBytes / 16;
  constexpr int kE = Chunk<T>::kElems;       // elements per 16-byte chunk
  constexpr int kRowChunks = DIM / kE;        // chunks per metadata row
  constexpr int kQuarter = DIM / 4;           // coordinates per wave
  constexpr int kQChunks = kQuarter / kE;

  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_phys[kTilePages];

  const int b = blockIdx.z, g = blockIdx.y;
  const int p0 = blockIdx.x * kTilePages;
  const int L = seq_len_clamped(seq_lens, b, D);
  const int np = n_pages_of(L, D.P);
  if (p0 >= np) return;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;

  if (tid < kTilePages) {
    const int p = p0 + tid;
    int ph = -1;
    if (p < np) {
      ph = page_table[(size_t)b * D.max_pages + p];
      if (ph < 0 || ph >= D.num_phys) ph = -1;
    }
    s_phys[tid] = ph;
  }
  __syncthreads();

  // ---- stage the tile's records in LDS (coalesced 16-byte loads)
  const char *mbase = reinterpret_cast<const char *>(meta);
  for (int c = tid; c < kTilePages * kRecChunks; c += kScoreThreads) {
    const int r = c / kRecChunks, off = c % kRecChunks;
    const int ph = s_phys[r];
    if (ph >= 0) {
      const uint4 v = *reinterpret_cast<const uint4 *>(
          mbase + ((size_t)ph * D.Hkv + g) * kRecBytes + (size_t)off * 16);
      *reinterpret_cast<uint4 *>(smem + r * kStride + off * 16) = v;
    }
  }
  __syncthreads();

  // ---- each wave: one coordinate quarter, lane = page
  double acc_b[G], acc_m[G], acc_v[G];
#pragma unroll
  for (int h = 0; h < G; ++h) acc_b[h] = acc_m[h] = acc_v[h] = 0.0;
  const double *cf = coef + ((size_t)(b * D.Hkv + g) * DIM) * G * 4;
  const unsigned char *rec = smem + lane * kStride;
#pragma unroll 1
  for (int qc = 0; qc < kQChunks; ++qc) {
    const int chunk = wave * kQChunks + qc;  // chunk index within a row
    double kmin[kE], kmax[kE], kmean[kE], kvar[kE];
    Chunk<T>::unpack(*reinterpret_cast<const uint4 *>(rec + (0 * kRowChunks + chunk) * 16), kmin);
    Chunk<T>::unpack(*reinterpret_cast<const uint4 *>(rec + (1 * kRowChunks + chunk) * 16), kmax);
    Chunk<T>::unpack(*reinterpret_cast<const uint4 *>(rec + (2 * kRowChunks + chunk) * 16), kmean);
    Chunk<T>::unpack(*reinterpret_cast<const uint4 *>(rec + (3 * kRowChunks + chunk) * 16), kvar);
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
  __syncthreads();  // the tile is no longer needed; reuse LDS for the reduction

  // red[w][k][lane], k = kind*G + h
  double *red = reinterpret_cast<double *>(smem);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    red[(wave * 3 * G + 0 * G + h) * kWave + lane] = acc_b[h];
    red[(wave * 3 * G + 1 * G + h) * kWave + lane] = acc_m[h];
    red[(wave * 3 * G + 2 * G + h) * kWave + lane] = acc_v[h];
  }
  __syncthreads();
  const double c = D.scale, c2 = D.scale * D.scale;
  for (int idx = tid; idx < 3 * G * kWave; idx += kScoreThreads) {
    const int k = idx / kWave, r = idx % kWave;
    const int p = p0 + r;
    if (p >= np) continue;
    double s = red[(0 * 3 * G + k) * kWave + r];
    s += red[(1 * 3 * G + k) * kWave + r];
    s += red[(2 * 3 * G + k) * kWave + r];
    s += red[(3 * 3 * G + k) * kWave + r];
    const int kind = k / G, h = g * G + (k % G);
    const size_t o = ((size_t)b * D.Hq + h) * D.max_pages + p;
    const bool ok = s_phys[r] >= 0;
    if (kind == 0) box[o] = ok ? __double2float_ru(c * s) : NAN;
    else if (kind == 1) mu[o] = ok ? (float)(c * s) : NAN;
    else var[o] = ok ? (float)(c2 * s) : NAN;
  }
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
  Carve cv(ws);
  double *coef = cv.take<double>((size_t)D.B * D.Hkv * D.d * D.G * 4);
  hipLaunchKernelGGL(score_coef_kernel<T>, dim3(D.B * D.Hkv), dim3(256), 0, s, D,
                     (const T *)q, coef);
  constexpr int kRecBytes = 4 * DIM * (int)sizeof(T);
  const size_t tile = (size_t)kTilePages * (kRecBytes + 16);
  const size_t red = (size_t)4 * 3 * G * kWave * sizeof(double);
  const size_t smem = tile > red ? tile : red;
  dim3 grid((D.max_pages + kTilePages - 1) / kTilePages, D.Hkv, D.B);
  hipLaunchKernelGGL((score_pages_kernel<T, DIM, G>), grid, dim3(kScoreThreads), smem, s, D,
                     (const T *)meta, page_table, seq_lens, coef, box, mu, var);
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

}  // namespace ekv
