// iso_softrank.h -- the soft rank with L2 regularization ("Merge Hulls Without Copying Vertices:
// GPU Isotonic Regression", Section 7.9, after Blondel et al.): theta = x / eps is projected onto
// the permutahedron of w = (n, ..., 1).  Per row: sort theta in decreasing order into s, fit the
// decreasing isotonic regression v of z = s - w (unit weights), and return r = s - v in the
// original order.
//
// Layout: the sort leaves perm[r * n + k] = the flat index of the element at sorted position k of
// row r.  z and v are fp64 arrays in sorted order; z is first rounded to the input type, so the
// fit solves the input precision's problem in fp64 and r is rounded once.
#pragma once

#include <rocprim/block/block_radix_sort.hpp>

#include "iso_geom.h"

namespace iso {

constexpr int kSrThreads = 256;

// Unsigned keys that sort ascending in the DEcreasing order of the values (NaN last for
// positive-signed NaN; a row holding a NaN is flagged by the fit anyway).
__device__ __forceinline__ uint32_t sr_key(float v) {
  const uint32_t b = (uint32_t)__float_as_uint(v);
  const uint32_t o = (b >> 31) ? ~b : (b | 0x80000000u);  // ascending order of v
  return ~o;
}
__device__ __forceinline__ uint64_t sr_key(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint64_t o = (b >> 63) ? ~b : (b | 0x8000000000000000ull);
  return ~o;
}

template <typename T, typename K>
__global__ __launch_bounds__(kSrThreads) void k_sr_keys(const T* __restrict__ x, int64_t N, K* __restrict__ keys) {
  const int64_t i = (int64_t)blockIdx.x * kSrThreads + threadIdx.x;
  if (i < N) keys[i] = sr_key(x[i]);
}

// fp32 values of several rows: 64-bit keys holding the row above the value's key, so that one
// stable sort orders by row, then by decreasing value, equal values keeping their column order.
__global__ __launch_bounds__(kSrThreads) void k_sr_row_keys(const float* __restrict__ x, int64_t N, int64_t n,
                                                            uint64_t* __restrict__ keys) {
  const int64_t i = (int64_t)blockIdx.x * kSrThreads + threadIdx.x;
  if (i < N) keys[i] = ((uint64_t)(i / n) << 32) | (uint64_t)sr_key(x[i]);
}

// Rows of at most kSrRowMax elements: one workgroup sorts a row in LDS (rocPRIM's block radix
// sort, stable, items in blocked order: thread t holds columns 8t .. 8t + 7, so equal keys keep
// their column order) and writes perm and z directly.
constexpr int kSrItems = 8;
constexpr int kSrRowMax = kSrThreads * kSrItems;

template <typename T, typename K>
__global__ __launch_bounds__(kSrThreads) void k_sr_row_sort(const T* __restrict__ x, int64_t n, double eps,
                                                            uint32_t* __restrict__ perm, double* __restrict__ z) {
  using Sort = rocprim::block_radix_sort<K, kSrThreads, kSrItems, uint32_t>;
  __shared__ typename Sort::storage_type st;
  const int64_t base = (int64_t)blockIdx.x * n;
  K keys[kSrItems];
  uint32_t cols[kSrItems];
#pragma unroll
  for (int k = 0; k < kSrItems; ++k) {
    const int c = threadIdx.x * kSrItems + k;
    keys[k] = c < n ? sr_key(x[base + c]) : ~(K)0;  // past the row: sorts last
    cols[k] = (uint32_t)c;
  }
  Sort().sort(keys, cols, st);
#pragma unroll
  for (int k = 0; k < kSrItems; ++k) {
    const int pos = threadIdx.x * kSrItems + k;
    if (pos < n) {
      const uint32_t c = cols[k];
      perm[base + pos] = (uint32_t)(base + c);
      const double s = (double)x[base + c] / eps;
      z[base + pos] = (double)(T)(s - (double)(n - pos));
    }
  }
}

// Row of each sorted element: the key of the second, stable pass that groups rows again.
__global__ __launch_bounds__(kSrThreads) void k_sr_rows(const uint32_t* __restrict__ idx, int64_t N, int64_t n,
                                                        uint32_t* __restrict__ rk) {
  const int64_t i = (int64_t)blockIdx.x * kSrThreads + threadIdx.x;
  if (i < N) rk[i] = (uint32_t)(idx[i] / (uint32_t)n);
}

// z_k = s_k - (n - k), rounded to T, as fp64; s_k = x[perm_k] / eps.
template <typename T>
__global__ __launch_bounds__(kSrThreads) void k_sr_problem(const T* __restrict__ x, const uint32_t* __restrict__ perm,
                                                           int64_t N, int64_t n, double eps,
                                                           double* __restrict__ z) {
  const int64_t i = (int64_t)blockIdx.x * kSrThreads + threadIdx.x;
  if (i >= N) return;
  const int64_t k = i % n;
  const double s = (double)x[perm[i]] / eps;
  z[i] = (double)(T)(s - (double)(n - k));
}

// r[perm_k] = s_k - v_k, rounded once to T.
template <typename T>
__global__ __launch_bounds__(kSrThreads) void k_sr_combine(const T* __restrict__ x, const uint32_t* __restrict__ perm,
                                                           const double* __restrict__ v, int64_t N, double eps,
                                                           T* __restrict__ r) {
  const int64_t i = (int64_t)blockIdx.x * kSrThreads + threadIdx.x;
  if (i >= N) return;
  const uint32_t p = perm[i];
  const double s = (double)x[p] / eps;
  r[p] = (T)(s - v[i]);
}

// u_k = g[perm_k] (the cotangent in sorted order), as fp64.
template <typename T>
__global__ __launch_bounds__(kSrThreads) void k_sr_gather(const T* __restrict__ g, const uint32_t* __restrict__ perm,
                                                          int64_t N, double* __restrict__ u) {
  const int64_t i = (int64_t)blockIdx.x * kSrThreads + threadIdx.x;
  if (i < N) u[i] = (double)g[perm[i]];
}

// The backward: r = s - v(s - w) with s a permutation of x / eps, so the cotangent of x is
// (u - A u) / eps put back in the original order, A the block averaging of the fit.
template <typename T>
__global__ __launch_bounds__(kSrThreads) void k_sr_grad(const double* __restrict__ u, const double* __restrict__ au,
                                                        const uint32_t* __restrict__ perm, int64_t N, double eps,
                                                        T* __restrict__ gx) {
  const int64_t i = (int64_t)blockIdx.x * kSrThreads + threadIdx.x;
  if (i < N) gx[perm[i]] = (T)((u[i] - au[i]) / eps);
}

}  // namespace iso
