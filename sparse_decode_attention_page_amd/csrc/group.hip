// group.hip -- group-shared page selection: one kept set per KV head, read once
// for the G query heads that share it.
//
// The selection policies of "Resumen Tecnico: EntmaxKV - Decodificacion
// Consciente del Soporte para Atencion Entmax" (gist.science/es/paper/
// 2605.21649, section 2.B) are stated per query.  With grouped-query attention
// the G heads of a KV head read the same pages, so one set per KV head lets the
// decode fetch each kept page once.  Readings (the summary leaves this open):
//  * Top-k: a page's group score is the largest box over the G heads (a NaN
//    box ranks below every number); the k pages with the largest group scores,
//    ties to the lower page index, listed ascending;
//  * Gaussian: a page is kept for the group iff at least one of the G heads
//    keeps it with its own tau-hat, margin and fallback page -- the largest
//    per-head margin (estimate minus threshold) is >= 0.
//
// Top-k runs the per-row radix selection on the per-page maxima (rows = KV
// heads); the Gaussian policy runs the per-head selector into the workspace and
// merges the G ascending lists per KV head through a flag per page.
#include "common.hpp"
#include "launch.hpp"

namespace ekv {

static Dims group_dims(const Dims &D) {
  Dims Dg = D;
  Dg.Hq = D.Hkv;
  Dg.G = 1;
  return Dg;
}

// gbox[(b Hkv + g) max_pages + p] = max over the group's heads of box (NaN only
// if every head's box is NaN), for p < N_b.
__global__ __launch_bounds__(256) void group_box_kernel(Dims D, const float *__restrict__ box,
                                                        const int32_t *__restrict__ seq_lens,
                                                        const uint8_t *__restrict__ seq_mask,
                                                        float *__restrict__ gbox) {
  const int gr = blockIdx.y, b = gr / D.Hkv, g = gr % D.Hkv;
  if (seq_mask && !seq_mask[b]) return;
  const int np = n_pages_of(seq_len_clamped(seq_lens, b, D), D.P);
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= np) return;
  float m = NAN;
  for (int h = 0; h < D.G; ++h) {
    const float x = box[((size_t)b * D.Hq + (size_t)g * D.G + h) * D.max_pages + p];
    if (x == x && !(m >= x)) m = x;  // skips NaN; m NaN takes any number
  }
  gbox[(size_t)gr * D.max_pages + p] = m;
}

// One block per (b, g): clear the page flags, mark the pages of the G heads'
// lists, write the marked pages in ascending order.  The flags are global
// workspace bytes written and read by this block only (ordered by the block's
// barriers).
__global__ __launch_bounds__(256) void group_union_kernel(Dims D, const int32_t *__restrict__ seq_lens,
                                                          const uint8_t *__restrict__ seq_mask,
                                                          const int32_t *__restrict__ hsel,
                                                          const int32_t *__restrict__ hcnt, uint8_t *flags,
                                                          int32_t *__restrict__ sel_idx,
                                                          int32_t *__restrict__ sel_cnt) {
  __shared__ int scan_scratch[256 / kWave];
  const int gr = blockIdx.x, b = gr / D.Hkv, g = gr % D.Hkv;
  if (seq_mask && !seq_mask[b]) return;
  const int np = n_pages_of(seq_len_clamped(seq_lens, b, D), D.P);
  const int tid = threadIdx.x;
  uint8_t *f = flags + (size_t)gr * D.max_pages;
  for (int p = tid; p < np; p += 256) f[p] = 0;
  __syncthreads();
  for (int h = 0; h < D.G; ++h) {
    const size_t r = (size_t)b * D.Hq + (size_t)g * D.G + h;
    const int c = min(max(hcnt[r], 0), np);
    for (int i = tid; i < c; i += 256) {
      const int p = hsel[r * D.max_pages + i];
      if (p >= 0 && p < np) f[p] = 1;
    }
  }
  __syncthreads();
  int listed = 0;
  int32_t *out = sel_idx + (size_t)gr * D.max_pages;
  for (int p0 = 0; p0 < np; p0 += 4 * 256) {
    const int pb = p0 + 4 * tid;
    int keep[4], mine = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      keep[u] = (pb + u < np) ? f[pb + u] : 0;
      mine += keep[u];
    }
    int tot;
    int at = listed + block_excl_scan(mine, scan_scratch, &tot);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (keep[u]) out[at++] = pb + u;
    listed += tot;
  }
  if (tid == 0) sel_cnt[gr] = listed;
}

// The same union with the page flags as a bitmap in LDS (one bit per page,
// set with LDS atomic OR), compacted in one pass: thread t owns a run of
// bitmap words, counts their bits, takes its first output slot from a block
// scan and writes its pages in ascending order.  For rows whose bitmap fits
// the LDS budget; group_union_kernel takes the others.
__global__ __launch_bounds__(256) void group_union_lds_kernel(Dims D, int words, const int32_t *__restrict__ seq_lens,
                                                              const uint8_t *__restrict__ seq_mask,
                                                              const int32_t *__restrict__ hsel,
                                                              const int32_t *__restrict__ hcnt,
                                                              int32_t *__restrict__ sel_idx,
                                                              int32_t *__restrict__ sel_cnt) {
  extern __shared__ unsigned int bm[];  // [words]
  __shared__ int scan_scratch[256 / kWave];
  const int gr = blockIdx.x, b = gr / D.Hkv, g = gr % D.Hkv;
  if (seq_mask && !seq_mask[b]) return;
  const int np = n_pages_of(seq_len_clamped(seq_lens, b, D), D.P);
  const int tid = threadIdx.x;
  for (int w = tid; w < words; w += 256) bm[w] = 0u;
  __syncthreads();
  for (int h = 0; h < D.G; ++h) {
    const size_t r = (size_t)b * D.Hq + (size_t)g * D.G + h;
    const int c = min(max(hcnt[r], 0), np);
    for (int i = tid; i < c; i += 256) {
      const int p = hsel[r * D.max_pages + i];
      if (p >= 0 && p < np) atomicOr(&bm[p >> 5], 1u << (p & 31));
    }
  }
  __syncthreads();
  const int per = (words + 255) / 256;
  const int w0 = min(tid * per, words), w1 = min(w0 + per, words);
  int mine = 0;
  for (int w = w0; w < w1; ++w) mine += __popc(bm[w]);
  int tot;
  int at = block_excl_scan(mine, scan_scratch, &tot);
  int32_t *out = sel_idx + (size_t)gr * D.max_pages;
  for (int w = w0; w < w1; ++w) {
    unsigned int bits = bm[w];
    while (bits) {
      out[at++] = w * 32 + (__ffs(bits) - 1);
      bits &= bits - 1u;
    }
  }
  if (tid == 0) sel_cnt[gr] = tot;
}

size_t topk_group_ws_bytes(const Dims &D) {
  Carve cv(nullptr);
  cv.take<float>((size_t)D.B * D.Hkv * D.max_pages);
  cv.take<char>(topk_ws_bytes(group_dims(D)));
  return cv.bytes();
}

hipError_t launch_topk_group(const Dims &D, const float *box, const int32_t *seq_lens, int k,
                             const uint8_t *seq_mask, int32_t *sel_idx, int32_t *sel_cnt, void *ws,
                             hipStream_t s) {
  const Dims Dg = group_dims(D);
  Carve cv(ws);
  float *gbox = cv.take<float>((size_t)D.B * D.Hkv * D.max_pages);
  void *tws = cv.take<char>(topk_ws_bytes(Dg));
  if (D.max_pages <= 0 || D.B * D.Hkv <= 0) return hipSuccess;
  dim3 grid((D.max_pages + 255) / 256, D.B * D.Hkv);
  hipLaunchKernelGGL(group_box_kernel, grid, dim3(256), 0, s, D, box, seq_lens, seq_mask, gbox);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topk(Dg, gbox, seq_lens, k, seq_mask, sel_idx, sel_cnt, tws, s);
}

size_t gauss_group_ws_bytes(const Dims &D) {
  Carve cv(nullptr);
  cv.take<char>(gauss_ws_bytes(D));
  cv.take<int32_t>((size_t)D.B * D.Hq * D.max_pages);
  cv.take<int32_t>((size_t)D.B * D.Hq);
  cv.take<uint8_t>((size_t)D.B * D.Hkv * D.max_pages);
  return cv.bytes();
}

hipError_t launch_gauss_group(const Dims &D, const float *box, const float *mu, const float *var,
                              const int32_t *seq_lens, double alpha, double delta, double n_sigma,
                              const uint8_t *seq_mask, int32_t *sel_idx, int32_t *sel_cnt, double *tau_hat,
                              void *ws, hipStream_t s) {
  Carve cv(ws);
  void *gws = cv.take<char>(gauss_ws_bytes(D));
  int32_t *hsel = cv.take<int32_t>((size_t)D.B * D.Hq * D.max_pages);
  int32_t *hcnt = cv.take<int32_t>((size_t)D.B * D.Hq);
  uint8_t *flags = cv.take<uint8_t>((size_t)D.B * D.Hkv * D.max_pages);
  hipError_t e = launch_gauss(D, box, mu, var, seq_lens, alpha, delta, n_sigma, seq_mask, hsel, hcnt, tau_hat,
                              gws, s);
  if (e != hipSuccess) return e;
  if (D.B * D.Hkv <= 0) return hipSuccess;
  const int words = (D.max_pages + 31) / 32;
  if ((size_t)words * 4 <= 48 * 1024)
    hipLaunchKernelGGL(group_union_lds_kernel, dim3(D.B * D.Hkv), dim3(256), (size_t)words * 4, s, D, words,
                       seq_lens, seq_mask, hsel, hcnt, sel_idx, sel_cnt);
  else
    hipLaunchKernelGGL(group_union_kernel, dim3(D.B * D.Hkv), dim3(256), 0, s, D, seq_lens, seq_mask, hsel, hcnt,
                       flags, sel_idx, sel_cnt);
  return hipGetLastError();
}

}  // namespace ekv
