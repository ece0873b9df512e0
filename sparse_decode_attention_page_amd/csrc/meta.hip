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

// One (page, KV head) record over the page's first n token slots, by the whole
// block: thread (tg, cp) owns coordinates 2cp and 2cp + 1 and the slots tg,
// tg + TG, ...; min/max fold in fp32 (exact), S1 = sum k and S2 = sum k^2 in
// fp64, then thread i < d combines the TG partials in group order and writes
// coordinate i of the record.  Slot `sub` (if >= 0) is read from `sub_row`
// instead of the page, so a row being written in the same launch is never read
// back.  Ends with a block barrier, so smem may be reused at once.
template <typename T, bool F8>
__device__ inline void page_record(const Dims &D, const T *__restrict__ kp, int n, int sub,
                                   const T *__restrict__ sub_row, int phys, int g, void *__restrict__ meta,
                                   unsigned char *smem) {
  const int d = D.d;
  const int half = d / 2;
  const int tg = threadIdx.x / half, cp = threadIdx.x % half;
  const int TG = blockDim.x / half;
  float *smin = reinterpret_cast<float *>(smem);
  float *smax = smin + TG * d;
  double *ss1 = reinterpret_cast<double *>(smax + TG * d);
  double *ss2 = ss1 + TG * d;
  float mn0 = INFINITY, mn1 = INFINITY, mx0 = -INFINITY, mx1 = -INFINITY;
  double s10 = 0.0, s11 = 0.0, s20 = 0.0, s21 = 0.0;
  for (int j = tg; j < n; j += TG) {
    const T *row = j == sub ? sub_row : kp + (size_t)j * d;
    float k0, k1;
    if constexpr (sizeof(T) == 2) {
      uint32_t w = reinterpret_cast<const uint32_t *>(row)[cp];
      k0 = bf16lo(w);
      k1 = bf16hi(w);
    } else {
      float2 w = reinterpret_cast<const float2 *>(row)[cp];
      k0 = w.x;
      k1 = w.y;
    }
    mn0 = fminf(mn0, k0); mx0 = fmaxf(mx0, k0);
    mn1 = fminf(mn1, k1); mx1 = fmaxf(mx1, k1);
    const double e0 = k0, e1 = k1;
    s10 += e0; s20 += e0 * e0;  // squares of bf16/fp32 values are exact in fp64
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
    double var = s2 / (double)n - __dmul_rn(mean, mean);  // mean^2 rounded on its own
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

static size_t page_record_smem(const Dims &D, int threads) {
  const int TG = threads / (D.d / 2);
  return (size_t)TG * D.d * (4 + 4 + 8 + 8);
}

template <typename T, bool F8>
__global__ __launch_bounds__(256) void build_meta_kernel(Dims D, const T *__restrict__ k_pool,
                                                         const int32_t *__restrict__ page_table,
                                                         const int32_t *__restrict__ seq_lens,
                                                         const int32_t *__restrict__ from_token,
                                                         void *__restrict__ meta) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int b = blockIdx.y, g = blockIdx.z;
  const int P = D.P;
  const int L = seq_len_clamped(seq_lens, b, D);
  const int np = n_pages_of(L, P);
  int first = 0;
  if (from_token) {
    int f = from_token[b];
    first = (f < 0 ? 0 : f) / P;
  }
  for (int p = first + blockIdx.x; p < np; p += gridDim.x) {
    const int phys = page_table[(size_t)b * D.max_pages + p];
    if (phys < 0 || phys >= D.num_phys) continue;  // uniform across the block
    const int n = min(P, L - p * P);
    const T *kp = k_pool + ((size_t)phys * D.Hkv + g) * (size_t)P * D.d;
    page_record<T, F8>(D, kp, n, -1, nullptr, phys, g, meta, smem);
  }
}

// Streaming upkeep: token L_b - 1 of every sequence b (seq_lens already count
// it) is written into its page slot, then that page's record is rebuilt over
// its filled slots -- the metadata kept current as pages fill.  One block per
// (b, g); threads i < d write element i of the new K and V rows, and the
// record takes the new slot's keys from k_new, so it equals a rebuild of the
// page by build_meta_kernel, bit for bit.
template <typename T, bool F8>
__global__ __launch_bounds__(256) void append_token_kernel(Dims D, const T *__restrict__ k_new,
                                                           const T *__restrict__ v_new, T *__restrict__ k_pool,
                                                           T *__restrict__ v_pool, const int32_t *__restrict__ page_table,
                                                           const int32_t *__restrict__ seq_lens, void *__restrict__ meta) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int b = blockIdx.x, g = blockIdx.y, d = D.d, P = D.P;
  const int L = seq_len_clamped(seq_lens, b, D);
  if (L <= 0) return;
  const int t = L - 1, p = t / P, slot = t - p * P;
  const int phys = page_table[(size_t)b * D.max_pages + p];
  if (phys < 0 || phys >= D.num_phys) return;  // uniform across the block
  const size_t pbase = ((size_t)phys * D.Hkv + g) * (size_t)P * d;
  const size_t nbase = ((size_t)b * D.Hkv + g) * (size_t)d;
  const int i = threadIdx.x;
  if (i < d) {
    k_pool[pbase + (size_t)slot * d + i] = k_new[nbase + i];
    v_pool[pbase + (size_t)slot * d + i] = v_new[nbase + i];
  }
  page_record<T, F8>(D, k_pool + pbase, slot + 1, slot, k_new + nbase, phys, g, meta, smem);
}

hipError_t launch_append_token(const Dims &D, int dtype, bool f8, const void *k_new, const void *v_new, void *k_pool,
                               void *v_pool, const int32_t *page_table, const int32_t *seq_lens, void *meta,
                               hipStream_t s) {
  if (D.B <= 0 || D.Hkv <= 0) return hipSuccess;
  dim3 grid(D.B, D.Hkv);
  const size_t smem = page_record_smem(D, 256);
  if (dtype == ENTMAXKV_BF16 && f8)
    hipLaunchKernelGGL((append_token_kernel<uint16_t, true>), grid, dim3(256), smem, s, D, (const uint16_t *)k_new,
                       (const uint16_t *)v_new, (uint16_t *)k_pool, (uint16_t *)v_pool, page_table, seq_lens, meta);
  else if (dtype == ENTMAXKV_BF16)
    hipLaunchKernelGGL((append_token_kernel<uint16_t, false>), grid, dim3(256), smem, s, D, (const uint16_t *)k_new,
                       (const uint16_t *)v_new, (uint16_t *)k_pool, (uint16_t *)v_pool, page_table, seq_lens, meta);
  else if (!f8)
    hipLaunchKernelGGL((append_token_kernel<float, false>), grid, dim3(256), smem, s, D, (const float *)k_new,
                       (const float *)v_new, (float *)k_pool, (float *)v_pool, page_table, seq_lens, meta);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_build_meta(const Dims &D, int dtype, bool f8, const void *k_pool, const int32_t *page_table,
                             const int32_t *seq_lens, const int32_t *from_token, void *meta,
                             hipStream_t s) {
  const int threads = 256;
  const size_t smem = page_record_smem(D, threads);
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
