// iso_ragged.h -- rows of unequal lengths, laid end to end ("Merge Hulls Without Copying Vertices:
// GPU Isotonic Regression", Section 9, Limitations: the fit takes a rectangular batch, and rows of
// unequal length are padded).
//
// A bucket of rows of similar lengths is copied into a rectangular [c, L] buffer.  After its last
// element each row is padded with a value beyond its own range (above its maximum for the
// increasing fit, below its minimum for the decreasing one) at unit weight.  Every block mean of
// the row's own fit lies within the row's range, so the pads never pool with the row's elements
// and its fit is unchanged: the hull of the padded diagram keeps the row's end point as a vertex,
// and the turns at it have the margin of the pad's distance from the range.  The padded bucket is
// fitted as a rectangular batch, and each row's own part of z and of the block starts is copied
// back.
#pragma once

#include "iso_geom.h"

namespace iso {

constexpr int kRagThreads = 256;
constexpr int kRagPer = 16;                          // elements per thread of a tile
constexpr int kRagTile = kRagThreads * kRagPer;      // elements per workgroup

// Unsigned keys ordered as the doubles they encode (NaN excluded by the callers).
__device__ __forceinline__ uint64_t ord_key(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}
__device__ __forceinline__ double ord_val(uint64_t k) {
  const uint64_t b = (k >> 63) ? (k & 0x7fffffffffffffffull) : ~k;
  return __longlong_as_double((long long)b);
}

// A bucket: c rows (row indices rows[0..c)), stride L elements in the padded buffers, each
// workgroup of the one-dimensional grid taking tile t of bucket row r (tiles = ceil(L / kRagTile)).
struct RagBucket {
  const int64_t* offs;  // [batch + 1] row offsets into the packed arrays
  const int64_t* rows;  // [c] the bucket's rows
  int64_t c;
  int64_t L;
  int64_t tiles;
};

__device__ __forceinline__ void rag_where(const RagBucket& B, int64_t& r, int64_t& t, int64_t& o,
                                          int64_t& len) {
  r = (int64_t)blockIdx.x / B.tiles;
  t = (int64_t)blockIdx.x - r * B.tiles;
  const int64_t row = B.rows[r];
  o = B.offs[row];
  len = B.offs[row + 1] - o;
}

// keys[r] := the key of the most negative (increasing) or most positive (decreasing) double,
// before the reduction below.
__global__ __launch_bounds__(kRagThreads) void k_rag_init(uint64_t* __restrict__ keys, int64_t c,
                                                          int dec) {
  const int64_t i = (int64_t)blockIdx.x * kRagThreads + threadIdx.x;
  if (i < c) keys[i] = dec ? ~0ull : 0ull;
}

// The row's maximum (increasing) or minimum (decreasing) over its non-NaN values, for rows that
// need pads (len < L).
template <typename T, bool D>
__global__ __launch_bounds__(kRagThreads) void k_rag_extreme(const T* __restrict__ y, RagBucket B,
                                                             uint64_t* __restrict__ keys) {
  int64_t r, t, o, len;
  rag_where(B, r, t, o, len);
  if (len >= B.L) return;
  const int64_t i0 = t * kRagTile;
  bool any = false;
  uint64_t best = D ? ~0ull : 0ull;
  for (int k = 0; k < kRagPer; ++k) {
    const int64_t i = i0 + (int64_t)k * kRagThreads + threadIdx.x;
    if (i < len) {
      const double v = (double)y[o + i];
      if (v == v) {
        const uint64_t kv = ord_key(v);
        best = D ? (kv < best ? kv : best) : (kv > best ? kv : best);
        any = true;
      }
    }
  }
  for (int s = 1; s < kWave; s <<= 1) {
    const uint64_t ob = __shfl_xor(best, s, kWave);
    best = D ? (ob < best ? ob : best) : (ob > best ? ob : best);
  }
  if (__any(any) && (threadIdx.x & (kWave - 1)) == 0) {
    if (D) atomicMin((unsigned long long*)&keys[r], (unsigned long long)best);
    else atomicMax((unsigned long long*)&keys[r], (unsigned long long)best);
  }
}

// Copies the bucket's rows into the padded [c, L] buffers and writes the pads.  With the row's
// extreme M, a pad is M + (|M| / 1024 + 1) (decreasing: M - (|M| / 1024 + 1)), rounded to T.
template <typename T, bool W, bool D>
__global__ __launch_bounds__(kRagThreads) void k_rag_pack(const T* __restrict__ y, const T* __restrict__ w,
                                                          RagBucket B, const uint64_t* __restrict__ keys,
                                                          T* __restrict__ yp, T* __restrict__ wp) {
  int64_t r, t, o, len;
  rag_where(B, r, t, o, len);
  const int64_t i0 = t * kRagTile;
  T pad = (T)0;
  if (len < B.L) {
    const double M = ord_val(keys[r]);
    const double step = fabs(M) * (1.0 / 1024.0) + 1.0;
    pad = (T)(D ? M - step : M + step);
  }
  T* yr = yp + r * B.L;
  T* wr = W ? wp + r * B.L : nullptr;
  for (int k = 0; k < kRagPer; ++k) {
    const int64_t i = i0 + (int64_t)k * kRagThreads + threadIdx.x;
    if (i < B.L) {
      if (i < len) {
        yr[i] = y[o + i];
        if (W) wr[i] = w[o + i];
      } else {
        yr[i] = pad;
        if (W) wr[i] = (T)1;
      }
    }
  }
}

// Copies each row's own part of the padded fit (and block starts) back, and its row flags.
template <typename T>
__global__ __launch_bounds__(kRagThreads) void k_rag_unpack(const T* __restrict__ zp,
                                                            const uint8_t* __restrict__ bp,
                                                            const uint32_t* __restrict__ fp, RagBucket B,
                                                            T* __restrict__ z, uint8_t* __restrict__ bstart,
                                                            uint32_t* __restrict__ rflags) {
  int64_t r, t, o, len;
  rag_where(B, r, t, o, len);
  const int64_t i0 = t * kRagTile;
  const T* zr = zp + r * B.L;
  const uint8_t* br = bp ? bp + r * B.L : nullptr;
  for (int k = 0; k < kRagPer; ++k) {
    const int64_t i = i0 + (int64_t)k * kRagThreads + threadIdx.x;
    if (i < len) {
      z[o + i] = zr[i];
      if (bstart) bstart[o + i] = br[i];
    }
  }
  if (t == 0 && threadIdx.x == 0) rflags[B.rows[r]] = fp[r];
}

// Row flags of every row := 0 (empty rows keep this).
__global__ __launch_bounds__(kRagThreads) void k_rag_clear_flags(uint32_t* __restrict__ f, int64_t batch) {
  const int64_t i = (int64_t)blockIdx.x * kRagThreads + threadIdx.x;
  if (i < batch) f[i] = 0u;
}

}  // namespace iso
