// meta.hip -- per-page key metadata ([EntmaxKV s.2.A], the lightweight
// per-page data the scorer reads instead of the keys).
//
// EntmaxKV s.2.A = section 2.A ("query-aware page scoring") of "Resumen Tecnico:
// EntmaxKV - Decodificacion Consciente del Soporte para Atencion Entmax",
// gist.science/es/paper/2605.21649.
//
// Record layout [phys][g][4][d]: k_min, k_max, mean, var.  One block builds one
// record: threads own a pair of coordinates and a stride of token slots, fold
// min/max in fp32 (exact) and S1 = sum k, S2 = sum k^2 in fp64 (exact for bf16
// keys), then a fixed-order tree over the token groups finishes the record.
//
// Compact records (bf16 keys): k_min bf16[d] | k_max bf16[d] | mean e4m3[d] |
// var e4m3[d], 6d bytes -- the same statistics with the Gaussian moments in
// OCP FP8 E4M3 (a quarter fewer bytes for the scorer to stream).
#include "common.hpp"
#include "launch.hpp"

namespace ekv {

// fp64 -> OCP FP8 E4M3 (bias 7, no infinities, largest finite 448): nearest,
// ties to even, magnitudes >= 448 saturate, NaN -> 0x7F.  The quantum is
// 2^(E-3) in the binade [2^E, 2^(E+1)) and 2^-9 below 2^-6; codes increase with
// the value, so code = 8(E + 7) + (r - 8) for the rounded significand r in
// [8, 16] (r = 16 moves to the next binade) and code = r in the subnormals.
__device__ inline uint8_t f64_to_e4m3(double x) {
  if (x != x) return 0x7F;
  const unsigned sg = __signbit(x) ? 0x80u : 0u;
  const double a = fabs(x);
  if (a >= 448.0) return (uint8_t)(sg | 0x7Eu);
  if (a == 0.0) return (uint8_t)sg;
  const int E = ilogb(a);
  const int qe = E < -6 ? -9 : E - 3;
  const int r = (int)rint(ldexp(a, -qe));
  const int code = qe == -9 ? r : 8 * (E + 7) + (r - 8);
  return (uint8_t)(sg | (unsigned)min(code, 0x7E));
}

template <typename T, bool F8>
__global__ __launch_bounds__(256) void build_meta_kernel(Dims D, const T *__restrict__ k_pool,
                                                         const int32_t *__restrict__ page_table,
                                                         const int32_t *__restrict__ seq_lens,
                                                         const int32_t *__restrict__ from_token,
                                                         void *__restrict__ meta) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int b = blockIdx.y, g = blockIdx.z;
  const int d = D.d, P = D.P;
  const int L = seq_len_clamped(seq_lens, b, D);
  const int np = n_pages_of(L, P);
  int first = 0;
  if (from_token) {
    int f = from_token[b];
    first = (f < 0 ? 0 : f) / P;
  }
  const int half = d / 2;
  const int tg = threadIdx.x / half, cp = threadIdx.x % half;
  const int TG = blockDim.x / half;
  float *smin = reinterpret_cast<float *>(smem);
  float *smax = smin + TG * d;
  double *ss1 = reinterpret_cast<double *>(smax + TG * d);
  double *ss2 = ss1 + TG * d;

  for (int p = first + blockIdx.x; p < np; p += gridDim.x) {
    const int phys = page_table[(size_t)b * D.max_pages + p];
    if (phys < 0 || phys >= D.num_phys) continue;  // uniform across the block
    const int n = min(P, L - p * P);
    const T *kp = k_pool + ((size_t)phys * D.Hkv + g) * (size_t)P * d;
    float mn0 = INFINITY, mn1 = INFINITY, mx0 = -INFINITY, mx1 = -INFINITY;
    double s10 = 0.0, s11 = 0.0, s20 = 0.0, s21 = 0.0;
    for (int j = tg; j < n; j += TG) {
      float k0, k1;
      if constexpr (sizeof(T) == 2) {
        uint32_t w = reinterpret_cast<const uint32_t *>(kp + (size_t)j * d)[cp];
        k0 = bf16lo(w);
        k1 = bf16hi(w);
      } else {
        float2 w = reinterpret_cast<const float2 *>(kp + (size_t)j * d)[cp];
        k0 = w.x;
        k1 = w.y;
      }
      mn0 = fminf(mn0, k0); mx0 = fmaxf(mx0, k0);
      mn1 = fminf(mn1, k1); mx1 = fmaxf(mx1, k1);
      const double e0 = k0, e1 = k1;
      s10 += e0; s20 += e0 * e0;
      s11 += e1; s21 += e1 * e1;
    }
    smin[tg * d + 2 * cp] = mn0; smin[tg * d + 2 * cp + 1] = mn1;
    smax[tg * d + 2 * cp] = mx0; smax[tg * d + 2 * cp + 1] = mx1;
    ss1[tg * d + 2 * cp] = s10; ss1[tg * d + 2 * cp + 1] = s11;
    ss2[tg * d + 2 * cp] = s20; ss2[tg * d + 2 * cp + 1] = s21;
    __syncthreads();
    if ((int)threadIdx.x < d) {
      const int i = threadIdx.x;
      float mn = smin[i], mx = smax[i];
      double s1 = ss1[i], s2 = ss2[i];
      for (int t = 1; t < TG; ++t) {
        mn = fminf(mn, smin[t * d + i]);
        mx = fmaxf(mx, smax[t * d + i]);
        s1 += ss1[t * d + i];
        s2 += ss2[t * d + i];
      }
      const double mean = s1 / (double)n;
      double var = s2 / (double)n - mean * mean;
      if (!(var > 0.0)) var = 0.0;
      if constexpr (F8) {
        unsigned char *rec = reinterpret_cast<unsigned char *>(meta) + ((size_t)phys * D.Hkv + g) * 6 * (size_t)d;
        store_rne<T>(reinterpret_cast<T *>(rec), 0 * d + i, (double)mn);
        store_rne<T>(reinterpret_cast<T *>(rec), 1 * d + i, (double)mx);
        rec[4 * d + i] = f64_to_e4m3(mean);
        rec[5 * d + i] = f64_to_e4m3(var);
      } else {
        T *rec = reinterpret_cast<T *>(meta) + ((size_t)phys * D.Hkv + g) * 4 * (size_t)d;
        store_rne<T>(rec, 0 * d + i, (double)mn);
        store_rne<T>(rec, 1 * d + i, (double)mx);
        store_rne<T>(rec, 2 * d + i, mean);
        store_rne<T>(rec, 3 * d + i, var);
      }
    }
    __syncthreads();
  }
}

hipError_t launch_build_meta(const Dims &D, int dtype, bool f8, const void *k_pool, const int32_t *page_table,
                             const int32_t *seq_lens, const int32_t *from_token, void *meta,
                             hipStream_t s) {
  const int threads = 256;
  const int TG = threads / (D.d / 2);
  const size_t smem = (size_t)TG * D.d * (4 + 4 + 8 + 8);
  // bulk: one block per page; append: a few blocks walk the rebuilt pages
  const int gx = from_token ? 4 : (D.max_pages < 65535 ? D.max_pages : 65535);
  dim3 grid(gx, D.B, D.Hkv);
  if (dtype == ENTMAXKV_BF16 && f8)
    hipLaunchKernelGGL((build_meta_kernel<uint16_t, true>), grid, dim3(threads), smem, s, D,
                       (const uint16_t *)k_pool, page_table, seq_lens, from_token, meta);
  else if (dtype == ENTMAXKV_BF16)
    hipLaunchKernelGGL((build_meta_kernel<uint16_t, false>), grid, dim3(threads), smem, s, D,
                       (const uint16_t *)k_pool, page_table, seq_lens, from_token, meta);
  else if (!f8)
    hipLaunchKernelGGL((build_meta_kernel<float, false>), grid, dim3(threads), smem, s, D,
                       (const float *)k_pool, page_table, seq_lens, from_token, meta);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ekv
