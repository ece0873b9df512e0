// softmax.hip -- full-cache softmax decode, the baseline the EntmaxKV summary
// measures its speedups against ("Resumen Tecnico: EntmaxKV ...", gist.science/
// es/paper/2605.21649, section 4, efficiency): exact softmax attention over every
// cached token with the same score scale.
//
// The whole K and V cache is streamed once, so the kernel is bound by HBM.
// Design (split-K, one pass):
//  * a block owns a KV head g of sequence b and a contiguous range of pages; all
//    G query heads of the group are served from the same K/V bytes;
//  * thread (token slot j, coordinate slice) loads its slice of K and V for slot j
//    of every page straight into registers (coalesced 16-byte loads, prefetched
//    one page ahead), so the main loop touches no LDS and has no barriers;
//  * each thread keeps a running softmax (max, sum, weighted V slice) per head
//    over "its" tokens and rescales only when its max grows;
//  * the running states are merged across slots (shuffles, then LDS) and written
//    per range; a small second launch merges the ranges of each query row in
//    range order.
//
// softmax_decode_sparse runs the same softmax over the kept pages of each query
// row only (the selection entmax_decode_sparse receives), so that entmax and
// softmax can be compared under one kept set (the summary's discarded-mass
// argument, section 3).  Selections differ between the query heads of a group,
// so a block serves one query row; the row's kept pages are dealt round-robin
// to a fixed number of ranges, so long and short selections both spread over
// blocks, and the merge launch combines the ranges in range order.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace ekv {

constexpr int kSThreads = 256;
constexpr int kMergeThreads = 256;  // merge: groups of DIM threads, each over every (256/DIM)-th partial

struct SoftmaxWs {
  float *part;              // [B][Hq][S][DIM + 2]  (m, l, acc[DIM]); l = NaN marks a bad page id
  int S;                    // ranges per (b, g), at most 1024
  int pps;                  // pages per range
};

template <typename T, int DIM, int P, int G>
__global__ __launch_bounds__(kSThreads) void softmax_decode_kernel(
    Dims D, const T *__restrict__ q, const T *__restrict__ k_pool, const T *__restrict__ v_pool,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ seq_lens, float *__restrict__ out,
    float *__restrict__ lse, SoftmaxWs ws) {
  constexpr int kParts = kSThreads / P;        // threads per token slot
  constexpr int kPer = DIM / kParts;           // coordinates per thread
  static_assert(kPer >= 2 && kPer % 2 == 0, "slice must hold bf16 pairs");
  constexpr int kWords = kPer * (int)sizeof(T) / 4;  // 32-bit words per slice
  __shared__ float xch[kSThreads / kWave][kParts][G][DIM / kParts + 2];

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int slot = tid / kParts, part = tid % kParts;
  const int L = seq_len_clamped(seq_lens, b, D);
  const int np = n_pages_of(L, P);
  const int p_begin = s * ws.pps, p_end = min(np, (s + 1) * ws.pps);

  float qv[G][kPer];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < kPer; ++e)
      qv[h][e] = load_f<T>(q, ((size_t)b * D.Hq + g * G + h) * DIM + part * kPer + e) * (float)D.scale;

  float m[G], l[G], acc[G][kPer];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < kPer; ++e) acc[h][e] = 0.0f;
  }

  auto slice_ptr = [&](const T *pool, int p) -> const uint32_t * {
    const int phys = page_table[(size_t)b * D.max_pages + p];
    return reinterpret_cast<const uint32_t *>(pool + (((size_t)phys * D.Hkv + g) * P + slot) * DIM + part * kPer);
  };
  auto page_ok = [&](int p) {
    const int phys = page_table[(size_t)b * D.max_pages + p];
    return phys >= 0 && phys < D.num_phys;
  };

  bool bad = false;
  uint32_t kw[kWords], vw[kWords];
  int p = p_begin;
  bool have = p < p_end && page_ok(p) && slot < min(P, L - p * P);
  if (p < p_end && !page_ok(p)) bad = true;
  if (have) {
    const uint32_t *kp = slice_ptr(k_pool, p), *vp = slice_ptr(v_pool, p);
#pragma unroll
    for (int w = 0; w < kWords; ++w) { kw[w] = kp[w]; vw[w] = vp[w]; }
  }
  for (; p < p_end; ++p) {
    // prefetch the next page's slices
    uint32_t nk[kWords], nv[kWords];
    const int pn = p + 1;
    bool have_n = false;
    if (pn < p_end) {
      if (!page_ok(pn)) bad = true;
      else if (slot < min(P, L - pn * P)) {
        have_n = true;
        const uint32_t *kp = slice_ptr(k_pool, pn), *vp = slice_ptr(v_pool, pn);
#pragma unroll
        for (int w = 0; w < kWords; ++w) { nk[w] = kp[w]; nv[w] = vp[w]; }
      }
    }
    if (have) {
      float kf[kPer], vf[kPer];
#pragma unroll
      for (int w = 0; w < kWords; ++w) {
        if constexpr (sizeof(T) == 2) {
          kf[2 * w] = bf16lo(kw[w]); kf[2 * w + 1] = bf16hi(kw[w]);
          vf[2 * w] = bf16lo(vw[w]); vf[2 * w + 1] = bf16hi(vw[w]);
        } else {
          kf[w] = __uint_as_float(kw[w]);
          vf[w] = __uint_as_float(vw[w]);
        }
      }
      float sc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = 0.0f;
#pragma unroll
        for (int e = 0; e < kPer; ++e) a = __builtin_fmaf(qv[h][e], kf[e], a);
        sc[h] = a;
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {  // full score of the token: sum over the slot's parts
#pragma unroll
        for (int o = kParts / 2; o > 0; o >>= 1) sc[h] += __shfl_xor(sc[h], o, kWave);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        if (sc[h] > m[h]) {
          const float r = __expf(m[h] - sc[h]);
          l[h] *= r;
#pragma unroll
          for (int e = 0; e < kPer; ++e) acc[h][e] *= r;
          m[h] = sc[h];
        }
        const float pw = __expf(sc[h] - m[h]);
        l[h] += pw;
#pragma unroll
        for (int e = 0; e < kPer; ++e) acc[h][e] = __builtin_fmaf(pw, vf[e], acc[h][e]);
      }
    }
    have = have_n;
#pragma unroll
    for (int w = 0; w < kWords; ++w) { kw[w] = nk[w]; vw[w] = nv[w]; }
  }

  // ---- merge the running states of the slots: within the wave (same part) ...
  constexpr int kSlotsPerWave = kWave / kParts;
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int o = kParts; o < kWave; o <<= 1) {
      const float mo = __shfl_xor(m[h], o, kWave), lo = __shfl_xor(l[h], o, kWave);
      const float mn = fmaxf(m[h], mo);
      const float ra = mn == -INFINITY ? 0.0f : __expf(m[h] - mn);
      const float rb = mn == -INFINITY ? 0.0f : __expf(mo - mn);
      l[h] = l[h] * ra + lo * rb;
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const float ao = __shfl_xor(acc[h][e], o, kWave);
        acc[h][e] = acc[h][e] * ra + ao * rb;
      }
      m[h] = mn;
    }
  }
  (void)kSlotsPerWave;
  // ... then across the waves through LDS
  const int wave = tid / kWave, lane = tid % kWave;
  if (lane < kParts) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      xch[wave][part][h][0] = m[h];
      xch[wave][part][h][1] = l[h];
#pragma unroll
      for (int e = 0; e < kPer; ++e) xch[wave][part][h][2 + e] = acc[h][e];
    }
  }
  __syncthreads();
  constexpr int kNW = kSThreads / kWave;
  float *dst = ws.part;
  for (int idx = tid; idx < G * DIM; idx += kSThreads) {
    const int h = idx / DIM, i = idx % DIM;
    const int pr = i / kPer, e = i % kPer;
    float mm = -INFINITY;
    for (int w = 0; w < kNW; ++w) mm = fmaxf(mm, xch[w][pr][h][0]);
    float ll = 0.0f, aa = 0.0f;
    for (int w = 0; w < kNW; ++w) {
      const float r = mm == -INFINITY ? 0.0f : __expf(xch[w][pr][h][0] - mm);
      ll += xch[w][pr][h][1] * r;
      aa += xch[w][pr][h][2 + e] * r;
    }
    float *rec = dst + (((size_t)b * D.Hq + g * G + h) * ws.S + s) * (DIM + 2);
    rec[2 + i] = aa;
    if (i == 0) { rec[0] = mm; rec[1] = bad ? NAN : ll; }
  }
}

// Merge the ranges of one query row in range order (a separate launch: plain
// cached loads of all ranges at once beat a last-block handoff here).
template <int DIM>
__global__ __launch_bounds__(kMergeThreads) void softmax_merge_kernel(Dims D, SoftmaxWs ws, float *__restrict__ out,
                                                                     float *__restrict__ lse) {
  // thread (grp, i): coordinate i of the partials r = grp, grp + kMergeGroups, ...
  // (loads issued 16 at a time); the groups' sums are combined in a fixed order
  constexpr int kMergeGroups = kMergeThreads / DIM;
  __shared__ float sm[1024], sf[1024], sl[1024];
  __shared__ float s_ll[kMergeGroups], s_aa[kMergeGroups][DIM];
  __shared__ float s_mm;
  __shared__ int s_nan;
  const int row = blockIdx.x, tid = threadIdx.x, grp = tid / DIM, i = tid % DIM;
  const int S = ws.S;
  const float *rec0 = ws.part + (size_t)row * S * (DIM + 2);
  for (int r = tid; r < S; r += kMergeThreads) {
    sm[r] = rec0[(size_t)r * (DIM + 2)];
    sl[r] = rec0[(size_t)r * (DIM + 2) + 1];
  }
  __syncthreads();
  if (tid == 0) {
    float mm = -INFINITY;
    int nan = 0;
    for (int r = 0; r < S; ++r) {
      mm = fmaxf(mm, sm[r]);
      nan |= sl[r] != sl[r];
    }
    s_mm = mm;
    s_nan = nan;
  }
  __syncthreads();
  const float mm = s_mm;
  for (int r = tid; r < S; r += kMergeThreads) sf[r] = sm[r] == -INFINITY ? 0.0f : __expf(sm[r] - mm);
  __syncthreads();
  float ll = 0.0f, aa = 0.0f;
#pragma unroll 1
  for (int r0 = grp; r0 < S; r0 += 16 * kMergeGroups) {
    float a[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int r = min(r0 + u * kMergeGroups, S - 1);
      a[u] = rec0[(size_t)r * (DIM + 2) + 2 + i];
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int r = r0 + u * kMergeGroups;
      if (r < S) {
        ll += sl[r] * sf[r];
        aa += a[u] * sf[r];
      }
    }
  }
  if (i == 0) s_ll[grp] = ll;
  s_aa[grp][i] = aa;
  __syncthreads();
  if (grp == 0) {
    float lt = s_ll[0], at = s_aa[0][i];
    for (int g = 1; g < kMergeGroups; ++g) { lt += s_ll[g]; at += s_aa[g][i]; }
    const size_t o = (size_t)row * DIM + i;
    if (s_nan) out[o] = NAN;
    else out[o] = lt > 0.0f ? at / lt : 0.0f;
    if (i == 0 && lse) lse[row] = s_nan ? NAN : (lt > 0.0f ? mm + logf(lt) : -INFINITY);
  }
}

static SoftmaxWs carve_softmax(const Dims &D, void *base, size_t *bytes) {
  SoftmaxWs w;
  const int bg = D.B * D.Hkv;
  int S = (1024 + bg - 1) / bg;
  const int maxS = (D.max_pages + 7) / 8;  // at least 8 pages per range
  if (S > maxS) S = maxS;
  if (S < 1) S = 1;
  w.S = S;
  w.pps = (D.max_pages + S - 1) / S;
  Carve cv(base);
  w.part = cv.take<float>((size_t)D.B * D.Hq * S * (D.d + 2));
  if (bytes) *bytes = cv.bytes();
  return w;
}

size_t softmax_ws_bytes(const Dims &D) {
  size_t b = 0;
  carve_softmax(D, nullptr, &b);
  return b;
}

template <typename T, int DIM, int P, int G>
static hipError_t launch_sm(const Dims &D, const void *q, const void *k, const void *v, const int32_t *pt,
                            const int32_t *sl, float *out, float *lse, SoftmaxWs w, hipStream_t s) {
  dim3 grid(w.S, D.Hkv, D.B);
  hipLaunchKernelGGL((softmax_decode_kernel<T, DIM, P, G>), grid, dim3(kSThreads), 0, s, D, (const T *)q,
                     (const T *)k, (const T *)v, pt, sl, out, lse, w);
  hipLaunchKernelGGL((softmax_merge_kernel<DIM>), dim3(D.B * D.Hq), dim3(kMergeThreads), 0, s, D, w, out, lse);
  return hipGetLastError();
}

template <typename T, int DIM, int P>
static hipError_t launch_sm_g(const Dims &D, const void *q, const void *k, const void *v, const int32_t *pt,
                              const int32_t *sl, float *out, float *lse, SoftmaxWs w, hipStream_t s) {
  switch (D.G) {
    case 1: return launch_sm<T, DIM, P, 1>(D, q, k, v, pt, sl, out, lse, w, s);
    case 2: return launch_sm<T, DIM, P, 2>(D, q, k, v, pt, sl, out, lse, w, s);
    case 4: return launch_sm<T, DIM, P, 4>(D, q, k, v, pt, sl, out, lse, w, s);
    case 8: return launch_sm<T, DIM, P, 8>(D, q, k, v, pt, sl, out, lse, w, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, int DIM>
static hipError_t launch_sm_p(const Dims &D, const void *q, const void *k, const void *v, const int32_t *pt,
                              const int32_t *sl, float *out, float *lse, SoftmaxWs w, hipStream_t s) {
  switch (D.P) {
    case 16: return launch_sm_g<T, DIM, 16>(D, q, k, v, pt, sl, out, lse, w, s);
    case 32: return launch_sm_g<T, DIM, 32>(D, q, k, v, pt, sl, out, lse, w, s);
    case 64: return launch_sm_g<T, DIM, 64>(D, q, k, v, pt, sl, out, lse, w, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_softmax(const Dims &D, int dtype, const void *q, const void *k_pool,
                          const void *v_pool, const int32_t *page_table, const int32_t *seq_lens,
                          float *out, float *lse, void *ws, hipStream_t s) {
  SoftmaxWs w = carve_softmax(D, ws, nullptr);
  if (dtype == ENTMAXKV_BF16) {
    if (D.d == 64) return launch_sm_p<uint16_t, 64>(D, q, k_pool, v_pool, page_table, seq_lens, out, lse, w, s);
    return launch_sm_p<uint16_t, 128>(D, q, k_pool, v_pool, page_table, seq_lens, out, lse, w, s);
  }
  if (D.d == 64) return launch_sm_p<float, 64>(D, q, k_pool, v_pool, page_table, seq_lens, out, lse, w, s);
  return launch_sm_p<float, 128>(D, q, k_pool, v_pool, page_table, seq_lens, out, lse, w, s);
}


// ------------------------------------------------ softmax over the kept pages
template <typename T, int DIM, int P>
__global__ __launch_bounds__(kSThreads) void softmax_sparse_kernel(
    Dims D, const T *__restrict__ q, const T *__restrict__ k_pool, const T *__restrict__ v_pool,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ sel_idx, const int32_t *__restrict__ sel_cnt, SoftmaxWs ws) {
  constexpr int kParts = kSThreads / P;
  constexpr int kPer = DIM / kParts;
  static_assert(kPer >= 2 && kPer % 2 == 0, "slice must hold bf16 pairs");
  constexpr int kWords = kPer * (int)sizeof(T) / 4;
  __shared__ float xch[kSThreads / kWave][kParts][DIM / kParts + 2];
  const int s = blockIdx.x, row = blockIdx.y;
  const int b = row / D.Hq, h = row % D.Hq, g = h / D.G;
  const int tid = threadIdx.x, slot = tid / kParts, part = tid % kParts;
  const int MP = D.max_pages;
  const int L = seq_len_clamped(seq_lens, b, D);
  const int np = n_pages_of(L, P);
  const int c_raw = sel_cnt[row];
  bool bad = c_raw < 0 || c_raw > np;  // a count outside [0, N_b] poisons the row
  const int cnt = bad ? 0 : c_raw;
  const int32_t *srow = sel_idx + (size_t)row * MP;

  float qv[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) qv[e] = load_f<T>(q, (size_t)row * DIM + part * kPer + e) * (float)D.scale;
  float m = -INFINITY, l = 0.0f, acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.0f;

  // item i of the row: its page must lie in [0, N_b), above the previous kept
  // page, with a valid physical page; returns the physical page or -1 (bad)
  auto item_phys = [&](int i, int &fill) -> int {
    const int p = srow[i];
    const int prev = i > 0 ? srow[i - 1] : -1;
    if (p < 0 || p >= np || p <= prev) return -1;
    const int ph = page_table[(size_t)b * MP + p];
    if (ph < 0 || ph >= D.num_phys) return -1;
    fill = min(P, L - p * P);
    return ph;
  };
  auto slice_ptr = [&](const T *pool, int ph) -> const uint32_t * {
    return reinterpret_cast<const uint32_t *>(pool + (((size_t)ph * D.Hkv + g) * P + slot) * DIM + part * kPer);
  };

  uint32_t kw[kWords], vw[kWords];
  int i = s;
  int fill = 0;
  int ph = i < cnt ? item_phys(i, fill) : -1;
  if (i < cnt && ph < 0) bad = true;
  bool have = ph >= 0 && slot < fill;
  if (have) {
    const uint32_t *kp = slice_ptr(k_pool, ph), *vp = slice_ptr(v_pool, ph);
#pragma unroll
    for (int w = 0; w < kWords; ++w) { kw[w] = kp[w]; vw[w] = vp[w]; }
  }
  for (; i < cnt; i += gridDim.x) {
    uint32_t nk[kWords], nv[kWords];
    const int in = i + gridDim.x;
    bool have_n = false;
    if (in < cnt) {
      int fn = 0;
      const int phn = item_phys(in, fn);
      if (phn < 0) bad = true;
      else if (slot < fn) {
        have_n = true;
        const uint32_t *kp = slice_ptr(k_pool, phn), *vp = slice_ptr(v_pool, phn);
#pragma unroll
        for (int w = 0; w < kWords; ++w) { nk[w] = kp[w]; nv[w] = vp[w]; }
      }
    }
    if (have) {
      float kf[kPer], vf[kPer];
#pragma unroll
      for (int w = 0; w < kWords; ++w) {
        if constexpr (sizeof(T) == 2) {
          kf[2 * w] = bf16lo(kw[w]); kf[2 * w + 1] = bf16hi(kw[w]);
          vf[2 * w] = bf16lo(vw[w]); vf[2 * w + 1] = bf16hi(vw[w]);
        } else {
          kf[w] = __uint_as_float(kw[w]);
          vf[w] = __uint_as_float(vw[w]);
        }
      }
      float sc = 0.0f;
#pragma unroll
      for (int e = 0; e < kPer; ++e) sc = __builtin_fmaf(qv[e], kf[e], sc);
#pragma unroll
      for (int o = kParts / 2; o > 0; o >>= 1) sc += __shfl_xor(sc, o, kWave);
      if (sc > m) {
        const float r = __expf(m - sc);
        l *= r;
#pragma unroll
        for (int e = 0; e < kPer; ++e) acc[e] *= r;
        m = sc;
      }
      const float pw = __expf(sc - m);
      l += pw;
#pragma unroll
      for (int e = 0; e < kPer; ++e) acc[e] = __builtin_fmaf(pw, vf[e], acc[e]);
    }
    have = have_n;
#pragma unroll
    for (int w = 0; w < kWords; ++w) { kw[w] = nk[w]; vw[w] = nv[w]; }
  }

  // merge the slots: within the wave (same part), then across waves through LDS
#pragma unroll
  for (int o = kParts; o < kWave; o <<= 1) {
    const float mo = __shfl_xor(m, o, kWave), lo = __shfl_xor(l, o, kWave);
    const float mn = fmaxf(m, mo);
    const float ra = mn == -INFINITY ? 0.0f : __expf(m - mn);
    const float rb = mn == -INFINITY ? 0.0f : __expf(mo - mn);
    l = l * ra + lo * rb;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const float ao = __shfl_xor(acc[e], o, kWave);
      acc[e] = acc[e] * ra + ao * rb;
    }
    m = mn;
  }
  const int wave = tid / kWave, lane = tid % kWave;
  if (lane < kParts) {
    xch[wave][part][0] = m;
    xch[wave][part][1] = l;
#pragma unroll
    for (int e = 0; e < kPer; ++e) xch[wave][part][2 + e] = acc[e];
  }
  const int any_bad = __syncthreads_or(bad ? 1 : 0);
  constexpr int kNW = kSThreads / kWave;
  float *rec = ws.part + ((size_t)row * ws.S + s) * (DIM + 2);
  for (int idx = tid; idx < DIM; idx += kSThreads) {
    const int pr = idx / kPer, e = idx % kPer;
    float mm = -INFINITY;
    for (int w = 0; w < kNW; ++w) mm = fmaxf(mm, xch[w][pr][0]);
    float ll = 0.0f, aa = 0.0f;
    for (int w = 0; w < kNW; ++w) {
      const float r = mm == -INFINITY ? 0.0f : __expf(xch[w][pr][0] - mm);
      ll += xch[w][pr][1] * r;
      aa += xch[w][pr][2 + e] * r;
    }
    rec[2 + idx] = aa;
    if (idx == 0) { rec[0] = mm; rec[1] = any_bad ? NAN : ll; }
  }
}

static SoftmaxWs carve_softmax_sparse(const Dims &D, void *base, size_t *bytes) {
  SoftmaxWs w;
  const int rows = D.B * D.Hq;
  int S = (2048 + rows - 1) / rows;  // about 2048 blocks
  if (S > 64) S = 64;
  if (S > D.max_pages) S = D.max_pages;
  if (S < 1) S = 1;
  w.S = S;
  w.pps = 0;  // ranges take every S-th kept page
  Carve cv(base);
  w.part = cv.take<float>((size_t)rows * S * (D.d + 2));
  if (bytes) *bytes = cv.bytes();
  return w;
}

size_t softmax_sparse_ws_bytes(const Dims &D) {
  size_t b = 0;
  carve_softmax_sparse(D, nullptr, &b);
  return b;
}

template <typename T, int DIM, int P>
static hipError_t launch_sms(const Dims &D, const void *q, const void *k, const void *v, const int32_t *pt,
                             const int32_t *sl, const int32_t *si, const int32_t *sc, float *out, float *lse,
                             SoftmaxWs w, hipStream_t s) {
  hipLaunchKernelGGL((softmax_sparse_kernel<T, DIM, P>), dim3(w.S, D.B * D.Hq), dim3(kSThreads), 0, s, D,
                     (const T *)q, (const T *)k, (const T *)v, pt, sl, si, sc, w);
  hipLaunchKernelGGL((softmax_merge_kernel<DIM>), dim3(D.B * D.Hq), dim3(kMergeThreads), 0, s, D, w, out, lse);
  return hipGetLastError();
}

template <typename T, int DIM>
static hipError_t launch_sms_p(const Dims &D, const void *q, const void *k, const void *v, const int32_t *pt,
                               const int32_t *sl, const int32_t *si, const int32_t *sc, float *out, float *lse,
                               SoftmaxWs w, hipStream_t s) {
  switch (D.P) {
    case 16: return launch_sms<T, DIM, 16>(D, q, k, v, pt, sl, si, sc, out, lse, w, s);
    case 32: return launch_sms<T, DIM, 32>(D, q, k, v, pt, sl, si, sc, out, lse, w, s);
    case 64: return launch_sms<T, DIM, 64>(D, q, k, v, pt, sl, si, sc, out, lse, w, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_softmax_sparse(const Dims &D, int dtype, const void *q, const void *k_pool, const void *v_pool,
                                 const int32_t *page_table, const int32_t *seq_lens, const int32_t *sel_idx,
                                 const int32_t *sel_cnt, float *out, float *lse, void *ws, hipStream_t s) {
  SoftmaxWs w = carve_softmax_sparse(D, ws, nullptr);
  if (dtype == ENTMAXKV_BF16) {
    if (D.d == 64) return launch_sms_p<uint16_t, 64>(D, q, k_pool, v_pool, page_table, seq_lens, sel_idx, sel_cnt, out, lse, w, s);
    return launch_sms_p<uint16_t, 128>(D, q, k_pool, v_pool, page_table, seq_lens, sel_idx, sel_cnt, out, lse, w, s);
  }
  if (D.d == 64) return launch_sms_p<float, 64>(D, q, k_pool, v_pool, page_table, seq_lens, sel_idx, sel_cnt, out, lse, w, s);
  return launch_sms_p<float, 128>(D, q, k_pool, v_pool, page_table, seq_lens, sel_idx, sel_cnt, out, lse, w, s);
}

}  // namespace ekv
