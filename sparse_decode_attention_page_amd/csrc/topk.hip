// topk.hip -- Top-k page selection ([EntmaxKV s.2.B], policy 1: a fixed budget
// of the k pages with the highest bounding-box bound).
//
// EntmaxKV s.2.B = section 2.B ("candidate selection policies") of "Resumen
// Tecnico: EntmaxKV - Decodificacion Consciente del Soporte para Atencion
// Entmax", gist.science/es/paper/2605.21649.
//
// One block per (b, h) row.  The bounds are mapped to order-preserving 32-bit
// keys and the k-th largest key is found by an MSB-first radix select (four
// 8-bit passes with an LDS histogram); a final ordered pass emits every page
// above that key plus the lowest-index pages equal to it, in ascending order.
// All of it is integer work, so the page set is exact.
//
// The row is taken in batches of kTopkThreads * kTopkPer pages, thread t
// holding pages [t kTopkPer, (t + 1) kTopkPer) of the batch in registers; a
// row of one batch (up to 16,384 pages) is read once and kept for every pass,
// longer rows read each batch again per pass.  In the histogram the lanes of a
// wave that share the leading lane's digit add with one atomic (the bounds of a
// row share their high bytes, so plain atomics would pile onto one or two
// bins), and each wave counts into its own histogram (no atomics across
// waves); the bin holding the k-th key comes from a scan over the 256 bins
// (summed over the waves); the emission takes two block scans per batch, since
// each thread's pages are consecutive.
#include "common.hpp"
#include "launch.hpp"

namespace ekv {

constexpr int kTopkThreads = 1024;
constexpr int kTopkPer = 16;
constexpr int kTopkBatch = kTopkThreads * kTopkPer;

// Adds each active lane's digit d to hist: the lanes sharing the lowest active
// lane's digit add with one atomic, the rest one by one.  (Measured on the 1M
// context: one aggregated group 22.9 us per top-k, two 24.7, four 28.0, none
// 31.5 -- further rounds cost more than the conflicts they remove.)
__device__ __forceinline__ void hist_add_wave(unsigned int *hist, unsigned int d, bool active) {
  const int lane = threadIdx.x & (kWave - 1);
  const unsigned long long act = __ballot(active);
  if (act != 0ull) {  // uniform
    const int leader = __ffsll((long long)act) - 1;
    const unsigned int dl = (unsigned int)__builtin_amdgcn_readlane((int)d, leader);
    const unsigned long long m = __ballot(active && d == dl) & act;
    if (lane == leader) atomicAdd(&hist[dl], (unsigned int)__popcll(m));
    if ((m >> lane) & 1ull) active = false;
  }
  if (active) atomicAdd(&hist[d], 1u);
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(Dims D, const float *__restrict__ box,
                                                            const int32_t *__restrict__ seq_lens, int k,
                                                            const uint8_t *__restrict__ seq_mask,
                                                            int32_t *__restrict__ sel_idx,
                                                            int32_t *__restrict__ sel_cnt) {
  constexpr int kNw = kTopkThreads / kWave;
  __shared__ unsigned int hist[kNw][256];  // one histogram per wave: no atomics across waves
  __shared__ int scan_scratch[kTopkThreads / kWave];
  __shared__ unsigned int bin_tot[256 / kWave];
  __shared__ unsigned int s_prefix, s_need;
  const int row = blockIdx.x;  // b*Hq + h
  const int b = row / D.Hq;
  if (seq_mask && !seq_mask[b]) return;
  const int L = seq_len_clamped(seq_lens, b, D);
  const int np = n_pages_of(L, D.P);
  const float *key_row = box + (size_t)row * D.max_pages;
  int32_t *out = sel_idx + (size_t)row * D.max_pages;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);

  if (np <= k) {
    for (int p = tid; p < np; p += kTopkThreads) out[p] = p;
    if (tid == 0) sel_cnt[row] = np;
    return;
  }
  const int nbat = (np + kTopkBatch - 1) / kTopkBatch;
  unsigned int key[kTopkPer];
  auto load = [&](int bat) __attribute__((always_inline)) {
    const int p0 = bat * kTopkBatch + tid * kTopkPer;
#pragma unroll
    for (int u = 0; u < kTopkPer; ++u) key[u] = p0 + u < np ? order_key(key_row[p0 + u]) : 0u;
  };
  if (nbat == 1) load(0);  // kept for every pass

  // ---- radix select of the k-th largest key
  unsigned int prefix = 0, pmask = 0, need = (unsigned int)k;
#pragma unroll 1
  for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
    for (int i = tid; i < kNw * 256; i += kTopkThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
#pragma unroll 1
    for (int bat = 0; bat < nbat; ++bat) {
      if (nbat > 1) load(bat);
      const int p0 = bat * kTopkBatch + tid * kTopkPer;
#pragma unroll
      for (int u = 0; u < kTopkPer; ++u)
        hist_add_wave(hist[tid / kWave], (key[u] >> shift) & 255u, p0 + u < np && (key[u] & pmask) == prefix);
    }
    __syncthreads();
    // thread t < 256 takes bin 255 - t: an inclusive scan over t gives the count
    // of keys in bins >= 255 - t; the bin where it reaches `need` holds the key
    unsigned int h = 0, x = 0;
    if (tid < 256) {  // waves 0 .. 3, whole
#pragma unroll
      for (int w = 0; w < kNw; ++w) h += hist[w][255 - tid];
      x = h;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const unsigned int y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
      }
      if (lane == kWave - 1) bin_tot[tid / kWave] = x;
    }
    __syncthreads();
    if (tid < 256) {
      unsigned int base = 0;
      for (int w = 0; w < tid / kWave; ++w) base += bin_tot[w];
      const unsigned int incl = base + x, excl = incl - h;
      if (excl < need && incl >= need) {
        s_prefix = prefix | ((unsigned int)(255 - tid) << shift);
        s_need = need - excl;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    need = s_need;
    pmask |= 255u << shift;
  }
  // prefix is the k-th largest key; take every key above it and the `need`
  // lowest-index keys equal to it, in index order, batch by batch
  const unsigned int T = prefix;
  int eq_before = 0, sel_before = 0;
#pragma unroll 1
  for (int bat = 0; bat < nbat; ++bat) {
    if (nbat > 1) load(bat);
    const int p0 = bat * kTopkBatch + tid * kTopkPer;
    int n_eq = 0;
#pragma unroll
    for (int u = 0; u < kTopkPer; ++u) n_eq += (p0 + u < np && key[u] == T) ? 1 : 0;
    int eq_total;
    int eq_rank = eq_before + block_excl_scan(n_eq, scan_scratch, &eq_total);
    unsigned int takem = 0;  // bit u: page p0 + u is taken
#pragma unroll
    for (int u = 0; u < kTopkPer; ++u) {
      const bool ok = p0 + u < np;
      const bool eq = ok && key[u] == T;
      if (ok && (key[u] > T || (eq && eq_rank < (int)need))) takem |= 1u << u;
      eq_rank += eq ? 1 : 0;
    }
    int sel_total;
    int pos = sel_before + block_excl_scan(__popc(takem), scan_scratch, &sel_total);
#pragma unroll
    for (int u = 0; u < kTopkPer; ++u)
      if ((takem >> u) & 1u) out[pos++] = p0 + u;
    eq_before += eq_total;
    sel_before += sel_total;
  }
  if (tid == 0) sel_cnt[row] = k;
}

size_t topk_ws_bytes(const Dims &) { return 0; }

hipError_t launch_topk(const Dims &D, const float *box, const int32_t *seq_lens, int k,
                       const uint8_t *seq_mask, int32_t *sel_idx, int32_t *sel_cnt, void *,
                       hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3(D.B * D.Hq), dim3(kTopkThreads), 0, s, D, box, seq_lens, k, seq_mask,
                     sel_idx, sel_cnt);
  return hipGetLastError();
}

}  // namespace ekv
