// common.hpp -- device helpers shared by the EntmaxKV HIP kernels (gfx950).
//
// Arithmetic contract used across the kernels (so that page sets and entmax
// supports agree bit for bit with an fp64 reference):
//  * bf16 x bf16 and bf16^2 x bf16 products carry <= 24 significant bits, so
//    they are exact in fp32 and in fp64; every dot product over a page record or
//    a key is summed in fp64 and rounded once when stored.
//  * The library is compiled with -ffp-contract=off; fused multiply-adds appear
//    only where written (__builtin_fma), i.e. where the product is exact.
//  * Every comparison that decides membership (page kept, token in support) is
//    made in fp64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "entmaxkv.h"

namespace ekv {

constexpr int kWave = 64;

// --------------------------------------------------------------------------- loads
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <typename T>
__device__ __forceinline__ float load_f(const T *p, size_t i);
template <>
__device__ __forceinline__ float load_f<uint16_t>(const uint16_t *p, size_t i) { return bf16_to_f32(p[i]); }
template <>
__device__ __forceinline__ float load_f<float>(const float *p, size_t i) { return p[i]; }

// N consecutive elements as floats with the widest loads that alignment allows:
// p must be aligned to min(16, N * sizeof(T)) bytes.
template <int N>
__device__ __forceinline__ void load_vec(const uint16_t *p, float (&v)[N]) {
  static_assert(N % 4 == 0, "bf16 vector loads take multiples of 4 elements");
  if constexpr (N % 8 == 0) {
#pragma unroll
    for (int c = 0; c < N / 8; ++c) {
      const uint4 u = reinterpret_cast<const uint4 *>(p)[c];
      v[8 * c + 0] = bf16lo(u.x); v[8 * c + 1] = bf16hi(u.x);
      v[8 * c + 2] = bf16lo(u.y); v[8 * c + 3] = bf16hi(u.y);
      v[8 * c + 4] = bf16lo(u.z); v[8 * c + 5] = bf16hi(u.z);
      v[8 * c + 6] = bf16lo(u.w); v[8 * c + 7] = bf16hi(u.w);
    }
  } else {
#pragma unroll
    for (int c = 0; c < N / 4; ++c) {
      const uint2 u = reinterpret_cast<const uint2 *>(p)[c];
      v[4 * c + 0] = bf16lo(u.x); v[4 * c + 1] = bf16hi(u.x);
      v[4 * c + 2] = bf16lo(u.y); v[4 * c + 3] = bf16hi(u.y);
    }
  }
}
template <int N>
__device__ __forceinline__ void load_vec(const float *p, float (&v)[N]) {
  static_assert(N % 4 == 0, "f32 vector loads take multiples of 4 elements");
#pragma unroll
  for (int c = 0; c < N / 4; ++c) {
    const float4 u = reinterpret_cast<const float4 *>(p)[c];
    v[4 * c + 0] = u.x; v[4 * c + 1] = u.y; v[4 * c + 2] = u.z; v[4 * c + 3] = u.w;
  }
}

// ----------------------------------------------------------------------- roundings
// fp64 -> bf16 round-to-nearest-even in one step: round to float with
// round-toward-zero plus a sticky bit (round-to-odd, exact enough because float
// carries 16 more bits than bf16), then round-to-nearest-even to bf16.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  if (x != x) return 0x7FC0;
  float t = __double2float_rz(x);
  uint32_t u = __float_as_uint(t);
  if ((double)t != x) u |= 1u;
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

template <typename T>
__device__ __forceinline__ void store_rne(T *p, size_t i, double x);
template <>
__device__ __forceinline__ void store_rne<uint16_t>(uint16_t *p, size_t i, double x) { p[i] = f64_to_bf16_rne(x); }
template <>
__device__ __forceinline__ void store_rne<float>(float *p, size_t i, double x) { p[i] = (float)x; }

// float -> uint32 whose unsigned order is the float order (NaN mapped to the
// lowest key, -0 mapped onto +0).
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f != f) return 0u;
  if (f == 0.0f) f = 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------- reductions
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    T w = __shfl_xor(v, o, kWave);
    v = w > v ? w : v;
  }
  return v;
}

// fp64 wave reductions on DPP: quad permutes and row rotates combine each row
// of 16 lanes inside the VALU, then the four row results are read out with
// readlane.  The order is fixed and the result is wave-uniform.  All 64 lanes
// must be active.
template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double v) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)u, kCtrl, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)(u >> 32), kCtrl, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)u, lane);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(u >> 32), lane);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
constexpr int kDppXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRor4 = 0x124;  // row_ror:4
constexpr int kDppRor8 = 0x128;  // row_ror:8
template <>
__device__ __forceinline__ double wave_sum<double>(double v) {
  v += dpp_f64<kDppXor1>(v);
  v += dpp_f64<kDppXor2>(v);
  v += dpp_f64<kDppRor4>(v);
  v += dpp_f64<kDppRor8>(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}
template <>
__device__ __forceinline__ int wave_sum<int>(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, kDppXor1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppXor2, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRor4, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRor8, 0xF, 0xF, false);
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}
template <>
__device__ __forceinline__ double wave_max<double>(double v) {
  v = fmax(v, dpp_f64<kDppXor1>(v));
  v = fmax(v, dpp_f64<kDppXor2>(v));
  v = fmax(v, dpp_f64<kDppRor4>(v));
  v = fmax(v, dpp_f64<kDppRor8>(v));
  return fmax(fmax(readlane_f64(v, 0), readlane_f64(v, 16)), fmax(readlane_f64(v, 32), readlane_f64(v, 48)));
}

// Block-wide sum with a deterministic order (waves combined in index order).
// `scratch` must hold blockDim.x / 64 values; result valid in every thread.
template <typename T>
__device__ __forceinline__ T block_sum(T v, T *scratch) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
  __syncthreads();
  T s = scratch[0];
  for (int i = 1; i < nw; ++i) s += scratch[i];
  return s;
}
// Two block sums for the price of one barrier pair; `scratch` holds
// 2 * blockDim.x / 64 values.
__device__ __forceinline__ void block_sum2(double &a, double &b, double *scratch) {
  a = wave_sum(a);
  b = wave_sum(b);
  const int w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) { scratch[w] = a; scratch[nw + w] = b; }
  __syncthreads();
  double sa = scratch[0], sb = scratch[nw];
  for (int i = 1; i < nw; ++i) { sa += scratch[i]; sb += scratch[nw + i]; }
  a = sa;
  b = sb;
}
// N block sums with one barrier pair; `scratch` holds N * blockDim.x / 64 values.
template <int N>
__device__ __forceinline__ void block_sum_n(double (&v)[N], double *scratch) {
  const int w = threadIdx.x / kWave, nw = blockDim.x / kWave;
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = wave_sum(v[i]);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0)
    for (int i = 0; i < N; ++i) scratch[i * nw + w] = v[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    double s = scratch[i * nw];
    for (int k = 1; k < nw; ++k) s += scratch[i * nw + k];
    v[i] = s;
  }
}
template <typename T>
__device__ __forceinline__ T block_max(T v, T *scratch) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
  __syncthreads();
  T s = scratch[0];
  for (int i = 1; i < nw; ++i) s = scratch[i] > s ? scratch[i] : s;
  return s;
}

// Block barrier: __syncthreads(), or (kLdsOnly) one that orders LDS accesses
// only and leaves the thread's global loads in flight (lds_barrier below).
template <bool kLdsOnly>
__device__ __forceinline__ void block_sync() {
  if constexpr (kLdsOnly) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else __syncthreads();
}

// Exclusive prefix sum over a block (int32), returns the total in *total.
// kLdsOnly: its barriers order LDS only (global loads issued before it stay
// in flight; the caller must not rely on it to order global memory).
template <bool kLdsOnly = false>
__device__ __forceinline__ int block_excl_scan(int v, int *scratch, int *total) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  block_sync<kLdsOnly>();
  if (lane == kWave - 1) scratch[w] = x;
  block_sync<kLdsOnly>();
  int base = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    if (i < w) base += scratch[i];
    tot += scratch[i];
  }
  *total = tot;
  return base + x - v;
}

// ------------------------------------------------------------------ phase marks
// EKV_MARK(kernel, phase) records the 100 MHz real-time clock per block and
// phase in builds compiled with -DEKV_TRACE (timeline analysis of a kernel's
// phases; each source file gets its own buffer and a dump function declared
// with EKV_TRACE_DUMP).  Without EKV_TRACE both compile to nothing.
#ifdef EKV_TRACE
static __device__ unsigned long long ekv_trace_buf[8][1 << 15][8];
#define EKV_MARK(K, PH)                                                                    \
  do {                                                                                     \
    if (threadIdx.x == 0)                                                                  \
      ekv_trace_buf[(K)][(blockIdx.x + gridDim.x * blockIdx.y) & ((1 << 15) - 1)][(PH)] =  \
          __builtin_amdgcn_s_memrealtime();                                                \
  } while (0)
#define EKV_TRACE_DUMP(NAME)                                                               \
  extern "C" int NAME(void *host) {                                                        \
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(ekv_trace_buf), sizeof(ekv_trace_buf)); \
  }                                                                                        \
  extern "C" int NAME##_clear() {                                                          \
    void *p = nullptr;                                                                     \
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(ekv_trace_buf)) != hipSuccess) return -1;        \
    return (int)hipMemset(p, 0, sizeof(ekv_trace_buf));                                    \
  }
#else
#define EKV_MARK(K, PH) \
  do {                  \
  } while (0)
#define EKV_TRACE_DUMP(NAME)
#endif

// --------------------------------------------------------------------- sequences
struct Dims {
  int B, Hq, Hkv, G, d, P, max_pages, num_phys;
  double scale;
};

__device__ __forceinline__ int seq_len_clamped(const int32_t *seq_lens, int b, const Dims &D) {
  long long L = seq_lens[b];
  long long cap = (long long)D.max_pages * D.P;
  if (L < 0) L = 0;
  if (L > cap) L = cap;
  return (int)L;
}
__device__ __forceinline__ int n_pages_of(int L, int P) { return (L + P - 1) / P; }

// Barrier that orders LDS accesses only.  __syncthreads() waits for every
// outstanding global load (vmcnt(0)), and so does a workgroup fence on LDS,
// since LDS-DMA loads (global_load_lds) count as LDS writes tracked by vmcnt;
// either would drain prefetches that are meant to stay in flight across the
// barrier.  This one waits for the wave's LDS operations only; the memory
// clobber keeps the compiler from moving memory accesses across it.  Data
// arriving by LDS-DMA must be waited for explicitly (vmcnt) before it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ----------------------------------------------------- cross-block handoff
// Data one block writes and another block of the SAME launch reads (partials
// handed to the "last block" of a group) goes through agent-scope relaxed
// atomic stores/loads.  On gfx950 these are plain sc1 global stores/loads that
// are coherent across the XCDs' L2 caches, so the handoff needs no
// __threadfence() -- which here compiles to an L2 write-back plus invalidate
// per block and costs microseconds.
template <typename T>
struct ident { using type = T; };
template <typename T>
__device__ __forceinline__ void st_agent(T *p, typename ident<T>::type v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_agent(const T *p) {
  return __hip_atomic_load(const_cast<T *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// "last block done" handshake: every block of a group calls this once after
// handing off its results with st_agent; exactly one block (the last) sees
// true and may then read them with ld_agent.  Each thread first waits for its
// own stores to complete; thread 0 then bumps the group counter.  The last
// block resets the counter so the workspace can be reused without a memset.
__device__ __forceinline__ bool arrive_last(unsigned int *counter, unsigned int expected, int *flag_smem) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned int prev = atomicAdd(counter, 1u);
    bool last = (prev + 1 == expected);
    if (last) atomicExch(counter, 0u);
    *flag_smem = last ? 1 : 0;
  }
  __syncthreads();
  return *flag_smem != 0;
}


}  // namespace ekv
