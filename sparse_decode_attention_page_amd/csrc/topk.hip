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
#include "common.hpp"
#include "launch.hpp"

namespace ekv {

constexpr int kTopkThreads = 1024;

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(Dims D, const float *__restrict__ box,
                                                            const int32_t *__restrict__ seq_lens,
                                                            int k, const uint8_t *__restrict__ seq_mask,
                                                            int32_t *__restrict__ sel_idx,
                                                            int32_t *__restrict__ sel_cnt) {
  __shared__ unsigned int hist[256];
  __shared__ int scan_scratch[kTopkThreads / kWave];
  __shared__ unsigned int s_prefix, s_need;
  const int row = blockIdx.x;  // b*Hq + h
  const int b = row / D.Hq;
  if (seq_mask && !seq_mask[b]) return;
  const int L = seq_len_clamped(seq_lens, b, D);
  const int np = n_pages_of(L, D.P);
  const float *key_row = box + (size_t)row * D.max_pages;
  int32_t *out = sel_idx + (size_t)row * D.max_pages;
  const int tid = threadIdx.x;

  if (np <= k) {
    for (int p = tid; p < np; p += kTopkThreads) out[p] = p;
    if (tid == 0) sel_cnt[row] = np;
    return;
  }

  // ---- radix select of the k-th largest key
  unsigned int prefix = 0, pmask = 0, need = (unsigned int)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    for (int p = tid; p < np; p += kTopkThreads) {
      const unsigned int key = order_key(key_row[p]);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      unsigned int above = 0;
      int dgt = 255;
      for (; dgt > 0; --dgt) {
        if (above + hist[dgt] >= need) break;
        above += hist[dgt];
      }
      s_prefix = prefix | ((unsigned int)dgt << shift);
      s_need = need - above;
    }
    __syncthreads();
    prefix = s_prefix;
    need = s_need;
    pmask |= 255u << shift;
    __syncthreads();
  }
  // prefix is the k-th largest key; take every key above it and the `need`
  // lowest-index keys equal to it.
  const unsigned int T = prefix;
  int eq_before = 0, sel_before = 0;
  for (int base = 0; base < np; base += kTopkThreads) {
    const int p = base + tid;
    unsigned int key = 0;
    if (p < np) key = order_key(key_row[p]);
    const int is_eq = (p < np && key == T) ? 1 : 0;
    int eq_total;
    const int eq_rank = eq_before + block_excl_scan(is_eq, scan_scratch, &eq_total);
    const int take = (p < np) && (key > T || (is_eq && eq_rank < (int)need));
    int sel_total;
    const int pos = sel_before + block_excl_scan(take, scan_scratch, &sel_total);
    if (take) out[pos] = p;
    eq_before += eq_total;
    sel_before += sel_total;
  }
  if (tid == 0) sel_cnt[row] = k;
}

size_t topk_ws_bytes(const Dims &) { return 0; }

hipError_t launch_topk(const Dims &D, const float *box, const int32_t *seq_lens, int k,
                       const uint8_t *seq_mask, int32_t *sel_idx, int32_t *sel_cnt, void *,
                       hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3(D.B * D.Hq), dim3(kTopkThreads), 0, s, D, box, seq_lens, k,
                     seq_mask, sel_idx, sel_cnt);
  return hipGetLastError();
}

}  // namespace ekv
