// iso_kernels.h -- HIP kernels of the isotonic fit for gfx950 (wave64).
//
// Pipeline ("Merge Hulls Without Copying Vertices: GPU Isotonic Regression", Section 3):
//   k_tiny          rows of at most 16 elements, four lanes per row: pool adjacent violators.
//   k_wave          batches of more than 256 rows of 17 to 2048 elements, packed L = 1, 2, .., 64
//                   lanes per row and 64 / L rows per wavefront (Section 3.5): coalesced 16-byte loads,
//                   double-double cumulative sums in LDS
//                   (lane-serial, then a wave scan of lane totals), lane hulls by the bit-mask
//                   monotone chain (Section 3.1), pairwise walks merging lane hulls (Section 3.2);
//                   writes z and block starts.
//   k_row           (iso_row.h) rows of 2049 to 4096 elements, and shorter rows in batches of at
//                   most 256: one row per workgroup of 1024 threads, candidate-parallel bridges.
//   k_chunk         (iso_chunk.h) the chunk pass of longer rows.
//   k_scan_reduce / k_scan_apply   double-double exclusive scan of the chunk totals: the chunk
//                   starts of the coordinate hierarchy (Section 3.3 and Section 6 "Coordinates").
//   k_merge_levels  (iso_merge.h) three levels of the merge tree per launch, one wavefront per merge.
//   k_ends          per chunk: its range of surviving vertices and the slopes into and out of it,
//                   by bisection over the root list (Section 3.4).
//   k_fit           per chunk: every element not already final gets the slope of the hull edge
//                   above it, rounded once to the output type (Section 3.4, Corollary 4.5).
//   k_vjp_*         block-averaging backward (Section 6 "Gradient").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "iso_geom.h"

namespace iso {

// ------------------------------------------------------------------ tile layout in LDS
// A tile of one wavefront holds R = 64 / L row segments of up to 32 L elements.  Row segment r's points
// 0..len occupy raw LDS indices r * (32 L + 1) + k; raw index i is stored at lds_pad(i) to
// spread a lane's 32 consecutive points over the banks.  Element i's increment (w_i, w_i y_i)
// is staged at the slot of its left point i and replaced by that point's coordinates.
constexpr int kRawPts = kWave * (kLanePts + 1);           // 2112 = max R (32 L + 1)
constexpr int kLdsPts = kRawPts + (kRawPts >> 5) + 8;     // padded
constexpr int kMaskWords = 2 * kWave + 8;                 // R (L + 1) <= 128

__device__ __forceinline__ int lds_pad(int i) { return i + (i >> 5); }

// 16-byte vectors of the element type.
template <typename T>
struct Vec16;
template <>
struct Vec16<float> {
  using type = float4;
  static constexpr int N = 4;
};
template <>
struct Vec16<double> {
  using type = double2;
  static constexpr int N = 2;
};

template <typename T>
__device__ __forceinline__ void vload(const T* p, T* out) {
  using V = typename Vec16<T>::type;
  const V v = *reinterpret_cast<const V*>(p);
  if constexpr (Vec16<T>::N == 4) {
    out[0] = v.x;
    out[1] = v.y;
    out[2] = v.z;
    out[3] = v.w;
  } else {
    out[0] = v.x;
    out[1] = v.y;
  }
}

template <typename T>
__device__ __forceinline__ void load16(const T* p, T* out) {
  vload(p, out);
}

template <typename T>
__device__ __forceinline__ void store16(T* p, const T* in) {
  using V = typename Vec16<T>::type;
  V v;
  if constexpr (Vec16<T>::N == 4) {
    v = V{in[0], in[1], in[2], in[3]};
  } else {
    v = V{in[0], in[1]};
  }
  *reinterpret_cast<V*>(p) = v;
}

// Nontemporal forms for data that a kernel reads or writes exactly once in a long stream: the
// hint keeps those lines from displacing reused ones in L2 and the last-level cache, and on gfx950
// it lets a read-once / write-once stream run measurably closer to HBM bandwidth.
template <typename T>
__device__ __forceinline__ void load16_nt(const T* p, T* out) {
  typedef T V __attribute__((ext_vector_type(Vec16<T>::N)));
  const V v = __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
#pragma unroll
  for (int k = 0; k < Vec16<T>::N; ++k) out[k] = v[k];
}

template <typename T>
__device__ __forceinline__ void store16_nt(T* p, const T* in) {
  typedef T V __attribute__((ext_vector_type(Vec16<T>::N)));
  V v;
#pragma unroll
  for (int k = 0; k < Vec16<T>::N; ++k) v[k] = in[k];
  __builtin_nontemporal_store(v, reinterpret_cast<V*>(p));
}

// A double moved across lanes by a DPP permutation within each row of 16 lanes (a VALU move, no
// LDS traffic).  Controls used: quad_perm [1,0,3,2] (0xB1) and [2,3,0,1] (0x4E) pair lanes at
// distance 1 and 2; row_half_mirror (0x141) pairs lane i with 7 - i of its eight; row_mirror
// (0x140) pairs lane i with 15 - i of its sixteen.  Applied in this order they combine, after k
// steps, every aligned group of 2^k lanes.
template <int CTRL>
__device__ __forceinline__ double dpp_move(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp((int)(b & 0xffffffffll), CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(b >> 32), CTRL, 0xf, 0xf, false);
  return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}

// One step of a butterfly sum of pairs (hi, lo): the partner's pair is added with the exact
// error of the hi addition kept in lo.  The sum is symmetric bit for bit, so both lanes of every
// step, and so every lane of the group at the end, hold the same pair.
template <int CTRL>
__device__ __forceinline__ DD dpp_pair_sum(DD a) {
  const DD b{dpp_move<CTRL>(a.hi), dpp_move<CTRL>(a.lo)};
  const DD s = two_sum(a.hi, b.hi);
  return DD{s.hi, (a.lo + b.lo) + s.lo};
}

// Sum of the pairs of each aligned group of G lanes (G = 2, 4, 8 or 16), in every lane of it.
template <int G>
__device__ __forceinline__ DD group_pair_sum(DD a) {
  if (G >= 2) a = dpp_pair_sum<0xB1>(a);
  if (G >= 4) a = dpp_pair_sum<0x4E>(a);
  if (G >= 8) a = dpp_pair_sum<0x141>(a);
  if (G >= 16) a = dpp_pair_sum<0x140>(a);
  return a;
}

// Elements per load tile of the chunk pass: 16 elements of each input per lane, 8 for weighted
// fp64 (the tile and its prefetched successor stay in registers).
template <typename T, bool W>
struct Tile {
  static constexpr int N = (W && sizeof(T) == 8) ? 8 : 16;
};

// q = e / d for 0 <= e < 8192, 1 <= d <= 8192 (float reciprocal, corrected to exact).
__device__ __forceinline__ int small_div(int e, int d, float inv) {
  int q = (int)((float)e * inv);
  if (q * d > e) --q;
  else if ((q + 1) * d <= e) ++q;
  return q;
}

template <bool W>
struct TilePts {
  const double* sX;
  const double* sY;
  int base;  // raw LDS index of point 0 of the row segment
  __device__ __forceinline__ void operator()(int k, double& x, double& y) const {
    int idx = lds_pad(base + k);
    x = W ? sX[idx] : (double)k;
    y = sY[idx];
  }
};

// The same points as pairs (x of an unweighted point is its index k0 + k, exact).
template <bool W>
struct TilePairs {
  const double* sX;
  const double* sY;
  const double* sXl;
  const double* sYl;
  int base;
  int k0;
  __device__ __forceinline__ PD operator()(int k) const {
    int idx = lds_pad(base + k);
    return PD{W ? DD{sX[idx], sXl[idx]} : DD{(double)(k0 + k), 0.0}, DD{sY[idx], sYl[idx]}};
  }
};

// Rows of 17 to 2048 elements.  Points are pairs (hi in sX/sY, lo in sXl/sYl): the lane's start,
// from a double-double scan of the lane totals, plus the lane's running sums.  A fast turn is
// used when it exceeds 2^-47 X Y, X the row's total weight (or length) and Y its sum of |w y|:
// every hi part is within u of its pair's magnitude (at most X or Y), so the fast turn of three
// points is within 26 u X Y of the turn of the pairs.  Slopes come from the pairs.
template <typename T, bool W, bool D>
__global__ __launch_bounds__(kWave) void k_wave(const T* __restrict__ y, const T* __restrict__ w,
                                                     T* __restrict__ z, uint8_t* __restrict__ bstart,
                                                     uint32_t* __restrict__ rflags, int64_t batch,
                                                     int64_t n, int Lpack) {
  constexpr bool EX = ExactProd<T, W>::value;
  constexpr int kThreads = kWave;
  constexpr int kPts = kLdsPts;
  constexpr int kMW = kMaskWords;
  __shared__ double sX[W ? kPts : 1];
  __shared__ double sY[kPts];
  __shared__ double sXl[W ? kPts : 1];
  __shared__ double sYl[kPts];
  __shared__ uint32_t sM[kMW];
  __shared__ int sLst[kMW], sFst[kMW];  // per mask word: last vertex at or before it, first at or after
  __shared__ uint32_t sF[kWave];

  constexpr int VN = Vec16<T>::N;
  const int lane = threadIdx.x;
  const int L = Lpack;
  const int R = kThreads / L;
  const int64_t row0 = (int64_t)blockIdx.x * R;
  const int64_t left = batch - row0;
  const int rows = left < R ? (int)left : R;
  const int64_t off = row0 * n;
  const int seglen = (int)n;
  const int rowStride = kLanePts * L + 1;
  const int maskStride = L + 1;
  const int E = rows * seglen;  // elements of the tile, contiguous from off
  const float inv_seg = 1.0f / (float)seglen;

  for (int i = lane; i < kMW; i += kThreads) sM[i] = 0u;
  if (lane < kWave) sF[lane] = 0u;

  // ---- a1: load.  All of the lane's loads are issued before any is used: 16-byte vectors at
  // element (lane + 64 k) * VN when the tile is 16-byte aligned, else scalars at lane + 64 k.
  T yv[kLanePts], wv[kLanePts];
  const bool vec = (((uintptr_t)(y + off)) % 16 == 0) && (!W || ((uintptr_t)(w + off)) % 16 == 0);
  if (vec) {
#pragma unroll
    for (int k = 0; k < kLanePts / VN; ++k) {
      const int e = (lane + kThreads * k) * VN;
      if (e + VN <= E) {
        vload(y + off + e, &yv[k * VN]);
        if (W) vload(w + off + e, &wv[k * VN]);
      } else {
#pragma unroll
        for (int t = 0; t < VN; ++t) {
          if (e + t < E) {
            yv[k * VN + t] = y[off + e + t];
            if (W) wv[k * VN + t] = w[off + e + t];
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < kLanePts; ++k) {
      const int e = lane + kThreads * k;
      if (e < E) {
        yv[k] = y[off + e];
        if (W) wv[k] = w[off + e];
      }
    }
  }
  __syncthreads();
  // classify and stage (w, w*y) in fp64 at each element's left point, with the product's
  // rounding error in the lo slot
#pragma unroll
  for (int k = 0; k < kLanePts; ++k) {
    const int e = vec ? (lane + kThreads * (k / VN)) * VN + (k % VN) : lane + kThreads * k;
    if (e < E) {
      double yd = yval<D>(yv[k]);
      double wd = W ? (double)wv[k] : 1.0;
      const int r = small_div(e, seglen, inv_seg);
      const int i = e - r * seglen;
      uint32_t f = 0u;
      if (!isfinite(yd) || !isfinite(wd)) f = ISO_ROW_NONFINITE_BIT;
      else if (!(wd > 0.0)) f = ISO_ROW_BAD_WEIGHT_BIT;
      if (f) {
        atomicOr(&sF[r], f);
        yd = 0.0;
        wd = 1.0;
      }
      const int slot = lds_pad(r * rowStride + i);
      if (W) sX[slot] = wd;
      const double p = wd * yd;
      sY[slot] = p;
      sYl[slot] = EX ? 0.0 : fma(wd, yd, -p);
    }
  }
  __syncthreads();

  // ---- a2: cumulative sums.  Lane-serial sums (pairs) of its 32 increments, a segmented
  // double-double scan of the lane totals, then each lane rewrites its slots with row-relative
  // pairs.
  const int lgL = __builtin_ctz(L);
  const int r2 = lane >> lgL;
  const int ql = lane & (L - 1);
  const bool rowOK = r2 < rows;
  int c = 0;
  if (rowOK) {
    int rem = seglen - kLanePts * ql;
    c = rem < 0 ? 0 : (rem > kLanePts ? kLanePts : rem);
  }
  const int rbase = r2 * rowStride;
  const int pbase = rbase + kLanePts * ql;
  const int nl = (seglen + kLanePts - 1) / kLanePts;  // active lanes of a row segment
  double Erow;  // the row's turn bound
  {
    DD tx{0.0, 0.0}, ty{0.0, 0.0};
    double ta = 0.0;
    for (int k = 0; k < kLanePts; ++k) {
      if (k < c) {
        const int idx = lds_pad(pbase + k);
        if (W) acc(tx.hi, tx.lo, sX[idx]);
        acc_pe(ty.hi, ty.lo, sY[idx], sYl[idx]);
        ta += fabs(sY[idx]);
      }
    }
    tx = two_sum(tx.hi, tx.lo);
    ty = two_sum(ty.hi, ty.lo);
    DD ix = tx, iy = ty, sx0, sy0;
    double xr = tx.hi, ar = ta;  // row sums of the lane totals (for the bound)
    for (int d = 1; d < L; d <<= 1) {
      const DD vx{__shfl_up(ix.hi, d, L), __shfl_up(ix.lo, d, L)};
      const DD vy{__shfl_up(iy.hi, d, L), __shfl_up(iy.lo, d, L)};
      if (ql >= d) {
        ix = dd_add(vx, ix);
        iy = dd_add(vy, iy);
      }
      xr += __shfl_xor(xr, d, L);
      ar += __shfl_xor(ar, d, L);
    }
    sx0 = DD{__shfl_up(ix.hi, 1, L), __shfl_up(ix.lo, 1, L)};
    sy0 = DD{__shfl_up(iy.hi, 1, L), __shfl_up(iy.lo, 1, L)};
    if (ql == 0) {
      sx0 = DD{0.0, 0.0};
      sy0 = DD{0.0, 0.0};
    }
    Erow = ((W ? xr : (double)seglen) * 0x1p-47) * ar;
    DD lx{0.0, 0.0}, ly{0.0, 0.0};
    for (int k = 0; k <= kLanePts; ++k) {
      // point k of the lane (the row segment's end point is written by its last active lane:
      // its slot belongs to no other lane's elements)
      if (k < c || (k == c && c > 0 && kLanePts * ql + c == seglen)) {
        const int idx = lds_pad(pbase + k);
        double rx = 0.0, ry = 0.0, rye = 0.0;
        if (k < c) {
          rx = W ? sX[idx] : 0.0;
          ry = sY[idx];
          rye = sYl[idx];
        }
        const PD P{W ? dd_add(sx0, lx) : DD{0.0, 0.0}, dd_add(sy0, ly)};
        if (W) {
          sX[idx] = P.x.hi;
          sXl[idx] = P.x.lo;
        }
        sY[idx] = P.y.hi;
        sYl[idx] = P.y.lo;
        if (W) acc(lx.hi, lx.lo, rx);
        acc_pe(ly.hi, ly.lo, ry, rye);
      }
    }
  }
  __syncthreads();

  // ---- a3: lane hulls.
  {
    TilePts<W> P{sX, sY, pbase};
    TilePairs<W> Q{sX, sY, sXl, sYl, pbase, kLanePts * ql};
    // x of an unweighted point is its row-local index.
    auto Pl = [&](int k, double& xx, double& yy) {
      P(k, xx, yy);
      if (!W) xx = (double)(kLanePts * ql + k);
    };
    uint64_t mk = lane_chain(c, Pl, Q, Erow);
    if (c > 0) {
      sM[r2 * maskStride + ql] = (uint32_t)mk;
      if (c == kLanePts && kLanePts * ql + c == seglen) sM[r2 * maskStride + ql + 1] = 1u;
    }
  }
  __syncthreads();

  // ---- a4: pairwise merges of lane hulls within each row segment, by walking.
  {
    TilePts<W> Prow{sX, sY, rbase};
    TilePairs<W> Qrow{sX, sY, sXl, sYl, rbase, 0};
    uint32_t* Mr = &sM[r2 * maskStride];
    for (int d = 1; d < L; d <<= 1) {
      if (rowOK && (ql & (2 * d - 1)) == 0 && ql + d < nl) {
        const int a0 = kLanePts * ql;
        const int s = kLanePts * (ql + d);
        int b1 = kLanePts * (ql + 2 * d);
        if (b1 > seglen) b1 = seglen;
        tile_walk_merge(Mr, a0, s, b1, Prow, Qrow, Erow);
      }
      __syncthreads();
    }
  }

  // ---- a5: emit.
  {
    // Per mask word of a row, the last vertex in the words up to it and the first in the words
    // from it on (a segmented max and min scan over the row's words), so that an element finds
    // the vertices around it with two lookups however far apart they are.
    constexpr int KW = (kMW + kThreads - 1) / kThreads;
    const int nwords = rows * maskStride;
    for (int p = lane; p < nwords; p += kThreads) {
      const uint32_t m = sM[p];
      const int u = p % maskStride;
      sLst[p] = m ? (u << 5) + 31 - __builtin_clz(m) : -1;
      sFst[p] = m ? (u << 5) + __builtin_ctz(m) : INT_MAX;
    }
    __syncthreads();
    for (int dd = 1; dd < maskStride; dd <<= 1) {
      int lv[KW], fv[KW];
#pragma unroll
      for (int t = 0; t < KW; ++t) {
        const int p = lane + t * kThreads;
        if (p < nwords) {
          const int u = p % maskStride;
          lv[t] = u >= dd ? max(sLst[p], sLst[p - dd]) : sLst[p];
          fv[t] = u + dd < maskStride ? min(sFst[p], sFst[p + dd]) : sFst[p];
        }
      }
      __syncthreads();
#pragma unroll
      for (int t = 0; t < KW; ++t) {
        const int p = lane + t * kThreads;
        if (p < nwords) {
          sLst[p] = lv[t];
          sFst[p] = fv[t];
        }
      }
      __syncthreads();
    }
    // Element-parallel: element e (row r, index i) gets the slope of the tile hull's edge over
    // it, from the vertex at or before point i to the vertex after it; an element whose two
    // points are both vertices is a block of its own and gets its y, the block's exact mean.
    // Consecutive lanes write consecutive elements.
    for (int e = lane; e < E; e += kThreads) {
      const T ye = y[off + e];  // issued first, so its latency overlaps the mask and LDS reads
      const int r = small_div(e, seglen, inv_seg);
      const int i = e - r * seglen;
      const uint32_t* Mr = &sM[r * maskStride];
      TilePairs<W> Qr{sX, sY, sXl, sYl, r * rowStride, 0};
      const int u = i >> 5, bt = i & 31;
      const uint32_t mw = Mr[u];
      const bool isv = (mw >> bt) & 1u;
      // point 0 is a vertex, so a word without a vertex at or before i is not the first one;
      // the row's end point is a vertex, so one without a vertex after i is not the last one
      const uint32_t ml = mw & (bt == 31 ? ~0u : ((2u << bt) - 1u));
      const uint32_t mh = bt == 31 ? 0u : (mw & ~((2u << bt) - 1u));
      const int a = ml ? (u << 5) + 31 - __builtin_clz(ml) : sLst[r * maskStride + u - 1];
      const int b = mh ? (u << 5) + __builtin_ctz(mh) : sFst[r * maskStride + u + 1];
      const bool bad = sF[r] != 0u;
      const double slope = slope_dd(Qr(a), Qr(b));
      z[off + e] = bad ? (T)NAN : (isv && b == i + 1) ? ye : (T)zval<D>(slope);
      if (bstart) bstart[off + e] = (!bad && isv) ? 1 : 0;
    }
    if (rowOK && ql == 0 && rflags) rflags[row0 + r2] = sF[r2];
  }
}

// ------------------------------------------------------------------ tiny rows
// Rows of at most kTinyMax elements, kTinyLanes lanes per row: pool adjacent violators, the
// classical sequential method the page names (Section 1), which for so few elements beats building
// the diagram's hull.  The row is cut into kTinyLanes parts of h = ceil(n / kTinyLanes) elements;
// each lane pools its part into a stack of blocks (the top block's fp64 sums (w, w*y) in
// registers, the blocks below it in LDS at their first element, the block starts in a bit mask).
// Then, in rounds, the first lane of each pair of neighbouring groups pushes the right group's
// blocks onto its stack in order, pooling while the block below has a mean >= the top one (means
// compared by cross-multiplication); a group's own blocks have increasing means, so once one of
// them is pushed without pooling the rest stay as they are.  The result is the pool adjacent
// violators fit of the whole row (pooling is order independent), its sums added in a different
// order than by one sequential scan.  The fit is each block's sum quotient rounded once, or y for
// a block of one element (its exact mean).
constexpr int kTinyMax = 16;
constexpr int kTinyLanes = 4;                        // lanes per row
constexpr int kTinyPart = kTinyMax / kTinyLanes;     // elements per lane at most
constexpr int kTinyRows = kWave / kTinyLanes;        // rows per wavefront

template <typename T, bool W, bool D>
__global__ __launch_bounds__(kWave) void k_tiny(const T* __restrict__ y, const T* __restrict__ w,
                                                T* __restrict__ z, uint8_t* __restrict__ bstart,
                                                uint32_t* __restrict__ rflags, int64_t batch, int n) {
  __shared__ double sS[kTinyMax][kTinyRows];
  __shared__ double sW[W ? kTinyMax : 1][kTinyRows];
  __shared__ uint32_t sMask[kTinyRows];
  const int lane = threadIdx.x;
  const int rr = lane / kTinyLanes;  // the row within the wavefront
  const int q = lane % kTinyLanes;   // the part of the row
  const int64_t row = (int64_t)blockIdx.x * kTinyRows + rr;
  const bool live = row < batch;
  const int hp = (n + kTinyLanes - 1) / kTinyLanes;
  const int h0 = min(q * hp, n);
  const int nh = min(hp, n - h0);
  const int64_t off = (live ? row : 0) * n + h0;
  constexpr int VN = Vec16<T>::N;
  // 16-byte vectors when every part is whole vectors at 16-byte aligned addresses
  const bool vec = (hp % VN) == 0 && (n % VN) == 0 && ((uintptr_t)y) % 16 == 0 && ((uintptr_t)z) % 16 == 0 &&
                   (!W || ((uintptr_t)w) % 16 == 0);
  T yv[kTinyPart], wv[kTinyPart];
  if (vec) {
#pragma unroll
    for (int k = 0; k < kTinyPart; k += VN) {
      if (live && k < nh) {
        load16(y + off + k, &yv[k]);
        if (W) load16(w + off + k, &wv[k]);
      }
    }
#pragma unroll
    for (int k = 0; k < kTinyPart; ++k) {
      if (!(live && k < nh)) {
        yv[k] = (T)0;
        wv[k] = (T)1;
      }
      if (!W) wv[k] = (T)1;
    }
  } else {
#pragma unroll
    for (int k = 0; k < kTinyPart; ++k) {
      yv[k] = (live && k < nh) ? y[off + k] : (T)0;
      wv[k] = (W && live && k < nh) ? w[off + k] : (T)1;
    }
  }
  uint32_t flag = 0u, mask = 0u;
  double tS = 0.0, tW = 1.0;
  int tt = h0;
  // pools the top block (tS, tW, tt) with the blocks below it while the one below has a mean >=
  // the top one's
  auto pool_down = [&]() {
    uint32_t below = mask & ~(1u << tt);
    while (below) {
      const int p = 31 - __builtin_clz(below);
      const double Sp = sS[p][rr], Wp = W ? sW[p][rr] : (double)(tt - p);
      if (!(Sp * tW >= tS * Wp)) break;
      tS = Sp + tS;
      tW = Wp + tW;
      tt = p;
      below &= ~(1u << p);
    }
    mask = below | (1u << tt);
  };
  // the lane's part: push element i as a block, then pool
#pragma unroll
  for (int k = 0; k < kTinyPart; ++k) {
    if (live && k < nh) {
      const int i = h0 + k;
      const double yd = yval<D>(yv[k]);
      const double wd = W ? (double)wv[k] : 1.0;
      if (!isfinite(yd) || !isfinite(wd)) flag |= ISO_ROW_NONFINITE_BIT;
      else if (!(wd > 0.0)) flag |= ISO_ROW_BAD_WEIGHT_BIT;
      const double Sn = wd * yd, Wn = wd;
      if (k > 0 && tS * Wn >= Sn * tW) {
        tS = tS + Sn;
        tW = tW + Wn;
        pool_down();
      } else {
        if (k > 0) {
          sS[tt][rr] = tS;
          if (W) sW[tt][rr] = tW;
        }
        mask |= 1u << i;
        tS = Sn;
        tW = Wn;
        tt = i;
      }
    }
  }
  if (live && nh > 0) {
    sS[tt][rr] = tS;
    if (W) sW[tt][rr] = tW;
  }
#pragma unroll
  for (int o = 1; o < kTinyLanes; o <<= 1) flag |= __shfl_xor(flag, o, kWave);
  // rounds: the group of lanes [q, q + 2 st) joins its right half [q + st, q + 2 st)
#pragma unroll
  for (int st = 1; st < kTinyLanes; st <<= 1) {
    const uint32_t mR = __shfl_down(mask, st, kWave);  // (used by the lanes with q % 2 st = 0)
    __syncthreads();
    if (live && q % (2 * st) == 0 && mR != 0u) {
      const int gend = min(h0 + 2 * st * hp, n);  // the right group's end
      uint32_t rest = mR;
      bool kept = false;
      while (rest) {
        const int p = __builtin_ctz(rest);
        rest &= rest - 1u;
        const int pe = rest ? __builtin_ctz(rest) : gend;  // the pushed block's end
        const double Sn = sS[p][rr], Wn = W ? sW[p][rr] : (double)(pe - p);
        if (!(tS * Wn >= Sn * tW)) {  // no pooling: this block and the rest stay as they are
          mask |= (1u << p) | rest;
          kept = true;
          break;
        }
        tS = tS + Sn;
        tW = tW + Wn;
        pool_down();
      }
      sS[tt][rr] = tS;
      if (W) sW[tt][rr] = tW;
      if (kept) {  // the joined group's top is the right group's last block
        tt = 31 - __builtin_clz(mask);
        tS = sS[tt][rr];
        tW = W ? sW[tt][rr] : (double)(gend - tt);
      }
    }
    __syncthreads();
  }
  if (live && q == 0) sMask[rr] = mask;
  __syncthreads();
  if (!live) return;
  const uint32_t fm = sMask[rr];
  // the fit: element i takes the mean of the block starting at the highest set bit <= i
  T zv[kTinyPart];
  uint8_t bs[kTinyPart];
#pragma unroll
  for (int k = 0; k < kTinyPart; ++k) {
    if (k < nh) {
      const int i = h0 + k;
      const int b = 31 - __builtin_clz(fm & ((2u << i) - 1u));
      const uint32_t after = fm & ~((2u << i) - 1u);  // block starts after i
      const int e = after ? __builtin_ctz(after) : n;  // end of i's block
      bs[k] = (b == i && !flag) ? 1 : 0;
      if (flag) zv[k] = (T)NAN;
      else if (e - b == 1) zv[k] = yv[k];
      else {
        const double Wb = W ? sW[b][rr] : (double)(e - b);
        zv[k] = (T)zval<D>(sS[b][rr] / Wb);
      }
    }
  }
  if (vec) {
#pragma unroll
    for (int k = 0; k < kTinyPart; k += VN)
      if (k < nh) store16(z + off + k, &zv[k]);
  } else {
#pragma unroll
    for (int k = 0; k < kTinyPart; ++k)
      if (k < nh) z[off + k] = zv[k];
  }
  if (bstart) {
#pragma unroll
    for (int k = 0; k < kTinyPart; ++k)
      if (k < nh) bstart[off + k] = bs[k];
  }
  if (rflags && q == 0) rflags[row] = flag;
}

// ------------------------------------------------------------------ chunk-start scan
constexpr int kScanThreads = 256;
constexpr int kScanPer = 4;
constexpr int kScanBlock = kScanThreads * kScanPer;  // chunks per scan block

struct DD2 {
  DD x, y;
};

__device__ __forceinline__ DD2 dd2_add(const DD2& a, const DD2& b) {
  return {dd_add(a.x, b.x), dd_add(a.y, b.y)};
}

// Inclusive block scan of DD2 values (Hillis-Steele in LDS).
__device__ __forceinline__ DD2 block_scan_incl(DD2 v, double* sh) {
  const int t = threadIdx.x;
  for (int d = 1; d < kScanThreads; d <<= 1) {
    sh[4 * t + 0] = v.x.hi;
    sh[4 * t + 1] = v.x.lo;
    sh[4 * t + 2] = v.y.hi;
    sh[4 * t + 3] = v.y.lo;
    __syncthreads();
    if (t >= d) {
      DD2 o{{sh[4 * (t - d) + 0], sh[4 * (t - d) + 1]}, {sh[4 * (t - d) + 2], sh[4 * (t - d) + 3]}};
      v = dd2_add(o, v);
    }
    __syncthreads();
  }
  return v;
}

__global__ __launch_bounds__(kScanThreads) void k_scan_reduce(const double2* __restrict__ tot,
                                                              const double2* __restrict__ totl,
                                                              const uint32_t* __restrict__ cflags,
                                                              double4* __restrict__ bsum,
                                                              uint32_t* __restrict__ bflag, int m,
                                                              int nblk) {
  __shared__ double sh[4 * kScanThreads];
  __shared__ uint32_t sf;
  const int64_t row = blockIdx.x / nblk;  // one-dimensional grid: batch * nblk blocks
  const int b = (int)(blockIdx.x - row * nblk);
  const int t = threadIdx.x;
  if (t == 0) sf = 0u;
  __syncthreads();
  DD2 acc{{0.0, 0.0}, {0.0, 0.0}};
  uint32_t f = 0u;
  for (int k = 0; k < kScanPer; ++k) {
    const int jj = b * kScanBlock + kScanPer * t + k;
    if (jj < m) {
      const double2 v = tot[row * m + jj], vl = totl[row * m + jj];
      acc = dd2_add(acc, DD2{{v.x, vl.x}, {v.y, vl.y}});
      f |= cflags[row * m + jj];
    }
  }
  if (f) atomicOr(&sf, f);
  DD2 incl = block_scan_incl(acc, sh);
  if (t == kScanThreads - 1) {
    bsum[row * nblk + b] = make_double4(incl.x.hi, incl.x.lo, incl.y.hi, incl.y.lo);
  }
  __syncthreads();
  if (t == 0) bflag[row * nblk + b] = sf;
}

// ONE: a row of at most kScanBlock chunks, scanned by this kernel alone (no block sums; the
// chunk flags are gathered here).
template <bool ONE>
__global__ __launch_bounds__(kScanThreads) void k_scan_apply(const double2* __restrict__ tot,
                                                             const double2* __restrict__ totl,
                                                             const double4* __restrict__ bsum,
                                                             const uint32_t* __restrict__ bflag,
                                                             const uint32_t* __restrict__ cflags,
                                                             double4* __restrict__ start,
                                                             uint32_t* __restrict__ rflags, int m,
                                                             int nblk) {
  __shared__ double sh[4 * kScanThreads];
  __shared__ double soff[4];
  __shared__ uint32_t sf;
  const int64_t row = blockIdx.x / nblk;  // one-dimensional grid: batch * nblk blocks
  const int b = (int)(blockIdx.x - row * nblk);
  const int t = threadIdx.x;
  if (ONE) {
    if (t == 0) {
      soff[0] = soff[1] = soff[2] = soff[3] = 0.0;
      sf = 0u;
    }
    __syncthreads();
    uint32_t f = 0u;
    for (int k = 0; k < kScanPer; ++k) {
      const int jj = kScanPer * t + k;
      if (jj < m) f |= cflags[row * m + jj];
    }
    if (f) atomicOr(&sf, f);
  } else if (t == 0) {
    DD2 o{{0.0, 0.0}, {0.0, 0.0}};
    uint32_t f = 0u;
    for (int k = 0; k < nblk; ++k) {
      const double4 v = bsum[row * nblk + k];
      if (k < b) o = dd2_add(o, DD2{{v.x, v.y}, {v.z, v.w}});
      f |= bflag[row * nblk + k];
    }
    soff[0] = o.x.hi;
    soff[1] = o.x.lo;
    soff[2] = o.y.hi;
    soff[3] = o.y.lo;
    if (b == 0 && rflags) rflags[row] = f;
  }
  DD2 loc[kScanPer + 1];
  loc[0] = DD2{{0.0, 0.0}, {0.0, 0.0}};
  for (int k = 0; k < kScanPer; ++k) {
    const int jj = b * kScanBlock + kScanPer * t + k;
    DD2 v{{0.0, 0.0}, {0.0, 0.0}};
    if (jj < m) {
      const double2 tv = tot[row * m + jj], tl = totl[row * m + jj];
      v = DD2{{tv.x, tl.x}, {tv.y, tl.y}};
    }
    loc[k + 1] = dd2_add(loc[k], v);
  }
  DD2 incl = block_scan_incl(loc[kScanPer], sh);  // (its barriers also publish soff and sf)
  if (ONE && t == 0 && rflags) rflags[row] = sf;
  // exclusive prefix of this thread = inclusive of the previous thread
  __syncthreads();
  sh[4 * t + 0] = incl.x.hi;
  sh[4 * t + 1] = incl.x.lo;
  sh[4 * t + 2] = incl.y.hi;
  sh[4 * t + 3] = incl.y.lo;
  __syncthreads();
  DD2 ex{{0.0, 0.0}, {0.0, 0.0}};
  if (t > 0) ex = DD2{{sh[4 * (t - 1) + 0], sh[4 * (t - 1) + 1]}, {sh[4 * (t - 1) + 2], sh[4 * (t - 1) + 3]}};
  const DD2 boff{{soff[0], soff[1]}, {soff[2], soff[3]}};
  const DD2 base = dd2_add(boff, ex);
  for (int k = 0; k < kScanPer; ++k) {
    const int jj = b * kScanBlock + kScanPer * t + k;
    if (jj < m) {
      const DD2 s = dd2_add(base, loc[k]);
      start[row * m + jj] = make_double4(s.x.hi, s.x.lo, s.y.hi, s.y.lo);
    }
  }
}

// ------------------------------------------------------------------ ends
template <typename T, bool W, bool D>
__global__ __launch_bounds__(256) void k_ends(VertexStore<T, W, D> S, EndInfo* __restrict__ ends,
                                              int64_t batch) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= batch * (int64_t)S.m) return;
  const int64_t row = g / S.m;
  ends[g] = chunk_ends(S, row, (int)(g - row * S.m));
}

// ------------------------------------------------------------------ fit
// nsub workgroups of 256 threads per chunk (nsub > 1 when there are too few chunks to fill the
// chip), element-parallel: the chunk's threads t = sub * 256 + tid take consecutive elements, or
// words, in turn.  Elements outside the chunk's surviving vertex range [klo, khi) lie under the edges
// into and out of it; inside it they lie under the chunk hull's own edges (Corollary 4.5).
//   list chunks:  the surviving vertices' point indices and the slopes between them are staged in
//                 LDS and each element finds its edge by binary search.
//   dense chunks: one thread walks each 32-element word once, carrying the lane's running sums
//                 from the word's checkpoint, so every point it passes costs one element's loads;
//                 at each vertex it writes the slope of the edge just closed to the elements
//                 under it.  An edge coming from an earlier word or going on to a later one costs
//                 one recomputation of that end point.  A one-element edge is its element's y,
//                 which the chunk pass already wrote in tiles where nothing was popped.
constexpr int kFitThreads = 256;
constexpr int kFitMaxSub = 4;  // workgroups per chunk at most

// Whether the chunk pass wrote z = y for element i (chunk-relative) of chunk g.
__device__ __forceinline__ bool ztile_set(const uint32_t* __restrict__ zt, int64_t g, int i) {
  return ((zt[g * kWave + i / kSub] >> ((i % kSub) / kZT)) & 1u) != 0u;
}
// The same from the chunk's marks staged in LDS (zl = its kWave words).
__device__ __forceinline__ bool ztile_set_l(const uint32_t* zl, int i) {
  return ((zl[i / kSub] >> ((i % kSub) / kZT)) & 1u) != 0u;
}

template <typename T, bool W, bool D>
__global__ __launch_bounds__(kFitThreads) void k_fit(VertexStore<T, W, D> S,
                                                     const EndInfo* __restrict__ ends,
                                                     const uint32_t* __restrict__ rflags,
                                                     const uint32_t* __restrict__ ztile,
                                                     T* __restrict__ z, uint8_t* __restrict__ bstart,
                                                     int nsub) {
  __shared__ double sSlope[kListCap];
  __shared__ int sK[kListCap];
  __shared__ uint32_t sMask[kMaskW];
  __shared__ uint32_t sZt[kWave];  // the chunk's z-tile marks (dense form)
  constexpr int TN = Tile<T, W>::N;
  const int64_t g = blockIdx.x / nsub;
  const int sub = (int)(blockIdx.x - g * nsub);
  const int64_t row = g / S.m;
  const int j = (int)(g - row * S.m);
  const int64_t off = row * S.n + (int64_t)j * kChunk;
  const int64_t rem = S.n - (int64_t)j * kChunk;
  const int len = rem < kChunk ? (int)rem : kChunk;
  const int tid = threadIdx.x;
  const int t0 = sub * kFitThreads + tid;  // this thread's rank among the chunk's threads
  const int tstride = nsub * kFitThreads;
  const EndInfo e = ends[g];
  // 16-byte groups of consecutive elements per thread (scalar stores where z is not aligned)
  constexpr int VN = Vec16<T>::N;
  const bool zvec = ((uintptr_t)(z + off)) % 16 == 0;
  auto fill = [&](const T zv, const bool start0) {
    T zo[VN];
#pragma unroll
    for (int u = 0; u < VN; ++u) zo[u] = zv;
    for (int i0 = t0 * VN; i0 < len; i0 += tstride * VN) {
      if (zvec && i0 + VN <= len) {
        store16(z + off + i0, zo);
      } else {
        for (int i = i0; i < min(i0 + VN, len); ++i) z[off + i] = zv;
      }
      if (bstart) {
        for (int i = i0; i < min(i0 + VN, len); ++i) bstart[off + i] = (i == 0 && start0) ? 1 : 0;
      }
    }
  };
  if (rflags[row] != 0u) {
    fill((T)NAN, false);
    return;
  }
  if (e.lo < 0) {
    fill((T)zval<D>(e.sin), e.p0v != 0);
    return;
  }
  // one-element blocks at the chunk's ends get their y: element 0 when P_0 is a vertex and P_1
  // the chunk's first surviving vertex, element len - 1 when P_{len-1} is the last surviving
  // vertex and P_len a vertex (the row's end, or the next chunk's point 0)
  const bool one_in = e.klo == 1 && e.p0v;
  const bool one_out = e.khi == len - 1 && (j + 1 == S.m || ends[g + 1].p0v);
  const T zin = one_in ? S.y[off] : (T)zval<D>(e.sin);
  const T zout = one_out ? S.y[off + len - 1] : (T)zval<D>(e.sout);
  if (S.dense[g] == 2 && e.khi == len && (e.klo == 0 || (e.klo == 1 && e.p0v))) {
    // every point of the chunk is a vertex of the chunk hull, and all of them are vertices of the
    // row's hull (point 0 possibly as the previous chunk's last vertex): every element is its own
    // block, and z = y was written for the whole chunk
    if (bstart) {
      for (int i = t0; i < len; i += tstride) bstart[off + i] = 1;
    }
    return;
  }
  if (!S.is_list(g)) {
    // a whole-diagram chunk (form 2) wrote z = y for every element and keeps no tile marks
    const bool zall = S.dense[g] == 2;
    for (int q = tid; q < kMaskW; q += kFitThreads) sMask[q] = S.mask[g * kMaskW + q];
    if (!zall)
      for (int q = tid; q < kWave; q += kFitThreads) sZt[q] = ztile[g * kWave + q];
    __syncthreads();
    // one word (32 elements) per thread at a time: a word inside [klo, khi) whose points and the
    // next one are all vertices, in tiles whose z the chunk pass wrote, needs nothing
    auto bit = [&](int i) { return ((sMask[i >> 5] >> (i & 31)) & 1u) != 0u; };
    const int nw = (len + 31) >> 5;
    // a word inside [klo, khi) whose points and the next one are all vertices holds blocks of
    // one element each, whose means are their y (Corollary 4.5): z = y where the chunk pass has
    // not written it yet, copied by all threads together in 16-byte groups (a group lies inside
    // one word and one z-tile mark)
    auto one_blocks = [&](int wd) {
      const int i0 = wd << 5, i1 = min(i0 + 32, len);
      return i0 >= e.klo && i1 <= e.khi && sMask[wd] == 0xffffffffu && (sMask[wd + 1] & 1u);
    };
    const bool yvec = zvec && ((uintptr_t)(S.y + off)) % 16 == 0;
    for (int i0 = t0 * VN; i0 < len; i0 += tstride * VN) {
      if (!one_blocks(i0 >> 5)) continue;
      const int n1 = min(VN, len - i0);
      if (bstart) {
        for (int u = 0; u < n1; ++u) bstart[off + i0 + u] = 1;
      }
      if (zall || ztile_set_l(sZt, i0)) continue;
      if (yvec && n1 == VN) {
        T v[VN];
        load16(S.y + off + i0, v);
        store16(z + off + i0, v);
      } else {
        for (int u = 0; u < n1; ++u) z[off + i0 + u] = S.y[off + i0 + u];
      }
    }
    for (int wd = t0; wd < nw; wd += tstride) {
      const int i0 = wd << 5;
      const int i1 = min(i0 + 32, len);
      if (one_blocks(wd)) continue;
      // elements before klo and from khi on lie under the edges into and out of the chunk
      for (int i = i0; i < min(i1, e.klo); ++i) {
        z[off + i] = zin;
        if (bstart) bstart[off + i] = (i == 0 && e.p0v) ? 1 : 0;
      }
      for (int i = max(i0, e.khi); i < i1; ++i) {
        z[off + i] = zout;
        if (bstart) bstart[off + i] = (i == e.khi) ? 1 : 0;
      }
      const int a0 = max(i0, e.klo), a1 = min(i1, e.khi);
      if (a0 >= a1) continue;
      // the edge (pa, b) covers the elements pa .. b - 1; its slope goes to those of them from
      // pend on inside this word (a later word holding more of the edge finds the same two
      // vertices and writes its own part; a one-element edge is its element's y, already written
      // where its tile is marked)
      auto close_edge = [&](int pend, int pa, const PD& Pa, int b, const PD& Pb) {
        if (b == pa + 1) {
          if (!zall && !ztile_set_l(sZt, pa)) z[off + pa] = S.y[off + pa];
          return;
        }
        const T zv = (T)zval<D>(slope_dd(Pa, Pb));
        const int stop = min(b, a1);
        for (int i = pend; i < stop; ++i) z[off + i] = zv;
      };
      DD sx, sy, ax, ay;
      S.dense_state(row, j, a0, sx, sy, ax, ay);
      int pa, pend = a0;
      PD Pa;
      if (bit(a0)) {
        pa = a0;
        Pa = S.join(sx, sy, ax, ay, a0);
      } else {
        pa = mask_pred(sMask, a0);
        Pa = S.dense_point(row, j, pa);
      }
      // the word's inputs are read four at a time, every read of a group issued before the
      // first one is used; the sums are taken in order, as before
      for (int i8 = a0; i8 < a1; i8 += 4) {
        T yg[4], wg[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          yg[k] = i8 + k < a1 ? S.y[off + i8 + k] : (T)0;
          wg[k] = (W && i8 + k < a1) ? S.w[off + i8 + k] : (T)1;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int i = i8 + k;
          if (i < a1) {
            double wd = W ? (double)wg[k] : 1.0;
            double yd = yval<D>(yg[k]);
            if (!isfinite(yd) || !isfinite(wd) || !(wd > 0.0)) {
              yd = 0.0;
              wd = 1.0;
            }
            if (bstart) bstart[off + i] = bit(i) ? 1 : 0;
            if (W) acc(ax.hi, ax.lo, wd);
            acc_prod<VertexStore<T, W, D>::EX>(ay.hi, ay.lo, wd, yd);
            const int ni = i + 1;
            if (ni < a1 && bit(ni)) {
              const PD Pb = S.join(sx, sy, ax, ay, ni);
              close_edge(pend, pa, Pa, ni, Pb);
              pa = ni;
              Pa = Pb;
              pend = ni;
            }
          }
        }
      }
      // the elements left lie under the edge from pa to the first vertex at or after a1: point a1
      // continues the walk unless it starts a word (a checkpoint) or ends the chunk
      const int b = bit(a1) ? a1 : mask_succ(sMask, a1);
      PD Pb;
      if (b == a1 && (a1 & (kCk - 1)) != 0 && a1 != len) {
        Pb = S.join(sx, sy, ax, ay, a1);
      } else {
        Pb = S.dense_point(row, j, b);
      }
      close_edge(pend, pa, Pa, b, Pb);
    }
    return;
  }
  // list form: stage the surviving vertices' point indices and the slopes of the edges between
  // them (a one-element edge's slope is its element's y, the block's exact mean)
  const int nv = e.hi - e.lo + 1;
  const int64_t lb = g * (int64_t)kListCap + e.lo;
  for (int q = tid; q < nv; q += kFitThreads) {
    const int k0 = S.lk[lb + q];
    sK[q] = k0;
    if (q + 1 < nv) {
      const int k1 = S.lk[lb + q + 1];
      sSlope[q] = k1 == k0 + 1 ? yval<D>(S.y[off + k0])
                               : slope_dd(PD{DD{S.lx[lb + q], S.lxl()[lb + q]}, DD{S.ly[lb + q], S.lyl()[lb + q]}},
                                          PD{DD{S.lx[lb + q + 1], S.lxl()[lb + q + 1]},
                                             DD{S.ly[lb + q + 1], S.lyl()[lb + q + 1]}});
    }
  }
  __syncthreads();
  // a thread takes VN consecutive elements: the first one inside [klo, khi) finds its edge by
  // binary search (edge q covers [sK[q], sK[q + 1])), the next ones step to the following edge
  // when they reach its first point
  for (int i0 = t0 * VN; i0 < len; i0 += tstride * VN) {
    T zo[VN];
    uint8_t so[VN];
    int q = -1;
#pragma unroll
    for (int u = 0; u < VN; ++u) {
      const int i = i0 + u;
      double zv = 0.0;
      uint8_t st = 0;
      if (i < e.klo) {
        zv = one_in ? yval<D>(S.y[off]) : e.sin;
        st = (i == 0 && e.p0v) ? 1 : 0;
      } else if (i >= e.khi) {
        if (i < len) zv = one_out ? yval<D>(S.y[off + i]) : e.sout;
        st = (i == e.khi) ? 1 : 0;
      } else {
        if (q < 0) {
          int lo = 0, hi = nv - 2;
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sK[mid] <= i) lo = mid;
            else hi = mid - 1;
          }
          q = lo;
        } else if (q + 1 <= nv - 2 && sK[q + 1] <= i) {
          ++q;
        }
        zv = sSlope[q];
        st = (sK[q] == i) ? 1 : 0;
      }
      zo[u] = (T)zval<D>(zv);
      so[u] = st;
    }
    if (zvec && i0 + VN <= len) {
      store16(z + off + i0, zo);
    } else {
#pragma unroll
      for (int u = 0; u < VN; ++u)
        if (i0 + u < len) z[off + i0 + u] = zo[u];
    }
    if (bstart) {
#pragma unroll
      for (int u = 0; u < VN; ++u)
        if (i0 + u < len) bstart[off + i0 + u] = so[u];
    }
  }
}

// ------------------------------------------------------------------ flags
__global__ __launch_bounds__(256) void k_flags_any(const uint32_t* __restrict__ rflags,
                                                   int64_t batch, uint32_t* __restrict__ any) {
  __shared__ uint32_t s;
  if (threadIdx.x == 0) s = 0u;
  __syncthreads();
  uint32_t f = 0u;
  for (int64_t i = threadIdx.x; i < batch; i += blockDim.x) f |= rflags[i];
  if (f) atomicOr(&s, f);
  __syncthreads();
  if (threadIdx.x == 0) any[0] = s;
}

// ------------------------------------------------------------------ backward (block averaging)
// With G and W the sums of g and w over the block holding element i, gy_i = w_i G / W and
// gw_i = (y_i - z_i) G / W.  For element i, G = F_i + R_i - g_i, where F_i sums g from its block's
// start to i (a left-to-right scan that restarts at every block start) and R_i from i to its
// block's end (a right-to-left scan that restarts after every block end); W likewise.  Tiles of
// kVjpTile elements, one workgroup of kVjpThreads threads each, kVjpPer2 consecutive elements
// per thread (coalesced loads); blocks crossing tiles get their sums from segmented scans of the
// tiles' head and tail sums.
constexpr int kVjpThreads = 256;
constexpr int kVjpPer2 = kVjpTile / kVjpThreads;

struct VjpTile {
  double hg, hw;  // sums before the tile's first block start (whole tile if none)
  double tg, tw;  // sums from the tile's last block start to its end (whole tile if none)
  int has;        // the tile holds a block start
  int pad;
};

struct Seg {
  int h;
  double g, w;
};

// left-to-right: a then b (a block start in b drops what a carried)
__device__ __forceinline__ Seg seg_lr(const Seg& a, const Seg& b) {
  return Seg{a.h | b.h, b.h ? b.g : a.g + b.g, b.h ? b.w : a.w + b.w};
}
// right-to-left: a (left) holds the fold of b (right) unless a holds a block start
__device__ __forceinline__ Seg seg_rl(const Seg& a, const Seg& b) {
  return Seg{a.h | b.h, a.h ? a.g : a.g + b.g, a.h ? a.w : a.w + b.w};
}

__device__ __forceinline__ Seg shfl_up_seg(const Seg& v, int d) {
  return Seg{__shfl_up(v.h, d, kWave), __shfl_up(v.g, d, kWave), __shfl_up(v.w, d, kWave)};
}
__device__ __forceinline__ Seg shfl_down_seg(const Seg& v, int d) {
  return Seg{__shfl_down(v.h, d, kWave), __shfl_down(v.g, d, kWave), __shfl_down(v.w, d, kWave)};
}

// Exclusive workgroup scans of one Seg per thread, in thread order: fw = fold of the threads
// before (left to right, seeded with fseed), bw = fold of the threads after (right to left,
// seeded with bseed).  sh: LDS of 2 * kVjpThreads / kWave Segs.
__device__ void vjp_wg_scans(Seg f, Seg r, const Seg& fseed, const Seg& bseed, Seg* sh, Seg& fw,
                             Seg& bw) {
  const int t = threadIdx.x, lane = t & (kWave - 1), wv = t >> 6;
  constexpr int NW = kVjpThreads / kWave;
  Seg fi = f, ri = r;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const Seg o = shfl_up_seg(fi, d);
    if (lane >= d) fi = seg_lr(o, fi);
    const Seg p = shfl_down_seg(ri, d);
    if (lane + d < kWave) ri = seg_rl(ri, p);
  }
  if (lane == kWave - 1) sh[wv] = fi;
  if (lane == 0) sh[NW + wv] = ri;
  __syncthreads();
  Seg fp = fseed;
  for (int k = 0; k < wv; ++k) fp = seg_lr(fp, sh[k]);
  Seg bp = bseed;
  for (int k = NW - 1; k > wv; --k) bp = seg_rl(sh[NW + k], bp);
  Seg fx = shfl_up_seg(fi, 1), rx = shfl_down_seg(ri, 1);
  fw = lane == 0 ? fp : seg_lr(fp, fx);
  bw = lane == kWave - 1 ? bp : seg_rl(rx, bp);
  __syncthreads();
}

template <typename T, bool NT = false>
__device__ __forceinline__ void vjp_load(const T* __restrict__ p, int64_t e0, int c, T (&v)[kVjpPer2],
                                         T fill) {
  constexpr int VN = Vec16<T>::N;
  if (c == kVjpPer2 && ((uintptr_t)(p + e0)) % 16 == 0) {
#pragma unroll
    for (int k = 0; k < kVjpPer2 / VN; ++k) {
      if constexpr (NT) load16_nt(p + e0 + k * VN, &v[k * VN]);
      else load16(p + e0 + k * VN, &v[k * VN]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < kVjpPer2; ++k) v[k] = k < c ? p[e0 + k] : fill;
  }
}

// Pass 1: each tile's head and tail sums.
template <typename T>
__global__ __launch_bounds__(kVjpThreads) void k_vjp_tiles(const T* __restrict__ g, const T* __restrict__ w,
                                                           const uint8_t* __restrict__ bs, int64_t n,
                                                           int ntile, VjpTile* __restrict__ tiles) {
  __shared__ Seg sh[2 * kVjpThreads / kWave];
  const int64_t tid = blockIdx.x;
  const int64_t row = tid / ntile;
  const int tt = (int)(tid - row * ntile);
  const int64_t off = row * n + (int64_t)tt * kVjpTile;
  const int64_t rem = n - (int64_t)tt * kVjpTile;
  const int len = rem < kVjpTile ? (int)rem : kVjpTile;
  const int i0 = kVjpPer2 * threadIdx.x;
  const int c = min(max(len - i0, 0), kVjpPer2);
  T gv[kVjpPer2], wv[kVjpPer2];
  vjp_load(g, off + i0, c, gv, (T)0);
  if (w) vjp_load(w, off + i0, c, wv, (T)0);
  int st[kVjpPer2];
  if (kVjpPer2 == 8 && c == kVjpPer2 && ((uintptr_t)(bs + off + i0)) % 8 == 0) {
    const uint64_t b8 = *reinterpret_cast<const uint64_t*>(bs + off + i0);
#pragma unroll
    for (int k = 0; k < kVjpPer2; ++k) st[k] = ((b8 >> (8 * k)) & 0xffu) ? 1 : 0;
  } else {
#pragma unroll
    for (int k = 0; k < kVjpPer2; ++k) st[k] = k < c ? (bs[off + i0 + k] ? 1 : 0) : 0;
  }
  // tail: left-to-right fold restarting at starts; head: sums before the first start
  Seg tl{0, 0.0, 0.0}, hd{0, 0.0, 0.0};
#pragma unroll
  for (int k = 0; k < kVjpPer2; ++k) {
    if (k < c) {
      const int b = st[k];
      const double gd = (double)gv[k], wd = w ? (double)wv[k] : 1.0;
      tl = seg_lr(tl, Seg{b, gd, wd});
      if (!hd.h && b) hd.h = 1;
      if (!hd.h) {
        hd.g += gd;
        hd.w += wd;
      }
    }
  }
  // The head fold is the right-to-left rule on (starts, sums before the first start): a thread
  // holding a start keeps only what precedes it.
  Seg fw, bw;
  vjp_wg_scans(tl, hd, Seg{0, 0.0, 0.0}, Seg{0, 0.0, 0.0}, sh, fw, bw);
  if (threadIdx.x == kVjpThreads - 1) {
    const Seg tot = seg_lr(fw, tl);
    tiles[tid].tg = tot.g;
    tiles[tid].tw = tot.w;
    tiles[tid].has = tot.h;
    tiles[tid].pad = 0;
  }
  if (threadIdx.x == 0) {
    const Seg tot = seg_rl(hd, bw);
    tiles[tid].hg = tot.g;
    tiles[tid].hw = tot.w;
  }
}

// Carries across tiles, per row: carry[t] = sums of the block open at tile t's start from earlier
// tiles (an exclusive left-to-right segmented scan of the tiles' tail sums) and cont[t] = sums of
// that block from tile t on (an inclusive right-to-left segmented scan of the tiles' head sums).
// The segmented rule, for a fold in either direction: (has, s) then (has', s') ->
// (has | has', has' ? s' : s + s') reading left to right, (has | has', has ? s : s + s') reading
// right to left.  Two passes over blocks of kVjpBlock tiles: each block's two folds, then each
// block combines the folds of the blocks before and after it and scans its own tiles.
constexpr int kVjpScanThreads = 256;
constexpr int kVjpPer = 4;
constexpr int kVjpBlock = kVjpScanThreads * kVjpPer;

// Inclusive block scan of Seg values: left to right (dir 1) or right to left (dir -1).
__device__ Seg vjp_block_scan(Seg v, int dir, int* sh_h, double* sh_g, double* sh_w) {
  const int t = threadIdx.x;
  for (int d = 1; d < kVjpScanThreads; d <<= 1) {
    sh_h[t] = v.h;
    sh_g[t] = v.g;
    sh_w[t] = v.w;
    __syncthreads();
    const int o = dir > 0 ? t - d : t + d;
    if (o >= 0 && o < kVjpScanThreads) {
      const Seg u{sh_h[o], sh_g[o], sh_w[o]};
      v = dir > 0 ? seg_lr(u, v) : seg_rl(v, u);
    }
    __syncthreads();
  }
  return v;
}

__global__ __launch_bounds__(kVjpScanThreads) void k_vjp_scan_reduce(const VjpTile* __restrict__ tiles,
                                                                    int ntile, int nblk,
                                                                    double4* __restrict__ bfw,
                                                                    double4* __restrict__ bbw) {
  __shared__ int sh_h[kVjpScanThreads];
  __shared__ double sh_g[kVjpScanThreads], sh_w[kVjpScanThreads];
  const int64_t row = blockIdx.x / nblk;  // one-dimensional grid: batch * nblk blocks
  const int b = (int)(blockIdx.x - row * nblk);
  const int t = threadIdx.x;
  const VjpTile* tr = tiles + row * ntile;
  Seg f{0, 0.0, 0.0}, r{0, 0.0, 0.0};
  for (int k = 0; k < kVjpPer; ++k) {
    const int tt = b * kVjpBlock + kVjpPer * t + k;
    if (tt < ntile) {
      const VjpTile v = tr[tt];
      f = seg_lr(f, Seg{v.has, v.tg, v.tw});
    }
  }
  for (int k = kVjpPer - 1; k >= 0; --k) {
    const int tt = b * kVjpBlock + kVjpPer * t + k;
    if (tt < ntile) {
      const VjpTile v = tr[tt];
      r = seg_rl(Seg{v.has, v.hg, v.hw}, r);
    }
  }
  f = vjp_block_scan(f, 1, sh_h, sh_g, sh_w);
  r = vjp_block_scan(r, -1, sh_h, sh_g, sh_w);
  if (t == kVjpScanThreads - 1) bfw[row * nblk + b] = make_double4(f.g, f.w, (double)f.h, 0.0);
  if (t == 0) bbw[row * nblk + b] = make_double4(r.g, r.w, (double)r.h, 0.0);
}

__global__ __launch_bounds__(kVjpScanThreads) void k_vjp_scan_apply(const VjpTile* __restrict__ tiles,
                                                                   int ntile, int nblk,
                                                                   const double4* __restrict__ bfw,
                                                                   const double4* __restrict__ bbw,
                                                                   double4* __restrict__ cc) {
  __shared__ int sh_h[kVjpScanThreads];
  __shared__ double sh_g[kVjpScanThreads], sh_w[kVjpScanThreads];
  __shared__ double soff[4];
  __shared__ int shas[2];
  const int64_t row = blockIdx.x / nblk;  // one-dimensional grid: batch * nblk blocks
  const int b = (int)(blockIdx.x - row * nblk);
  const int t = threadIdx.x;
  const VjpTile* tr = tiles + row * ntile;
  if (t == 0) {
    Seg pf{0, 0.0, 0.0};
    for (int k = 0; k < b; ++k) {
      const double4 v = bfw[row * nblk + k];
      pf = seg_lr(pf, Seg{(int)v.z, v.x, v.y});
    }
    Seg pb{0, 0.0, 0.0};
    for (int k = nblk - 1; k > b; --k) {
      const double4 v = bbw[row * nblk + k];
      pb = seg_rl(Seg{(int)v.z, v.x, v.y}, pb);
    }
    soff[0] = pf.g;
    soff[1] = pf.w;
    soff[2] = pb.g;
    soff[3] = pb.w;
    shas[0] = pf.h;
    shas[1] = pb.h;
  }
  // this thread's tiles, its left-to-right fold and its right-to-left fold
  Seg tv[kVjpPer], hv[kVjpPer];
  Seg f{0, 0.0, 0.0}, r{0, 0.0, 0.0};
  for (int k = 0; k < kVjpPer; ++k) {
    const int tt = b * kVjpBlock + kVjpPer * t + k;
    tv[k] = Seg{0, 0.0, 0.0};
    hv[k] = Seg{0, 0.0, 0.0};
    if (tt < ntile) {
      const VjpTile v = tr[tt];
      tv[k] = Seg{v.has, v.tg, v.tw};
      hv[k] = Seg{v.has, v.hg, v.hw};
    }
    f = seg_lr(f, tv[k]);
  }
  for (int k = kVjpPer - 1; k >= 0; --k) r = seg_rl(hv[k], r);
  const Seg fi = vjp_block_scan(f, 1, sh_h, sh_g, sh_w);
  const Seg ri = vjp_block_scan(r, -1, sh_h, sh_g, sh_w);
  // exclusive: the neighbouring thread's inclusive value
  sh_h[t] = fi.h;
  sh_g[t] = fi.g;
  sh_w[t] = fi.w;
  __syncthreads();
  Seg fe = Seg{shas[0], soff[0], soff[1]};
  if (t > 0) fe = seg_lr(fe, Seg{sh_h[t - 1], sh_g[t - 1], sh_w[t - 1]});
  __syncthreads();
  sh_h[t] = ri.h;
  sh_g[t] = ri.g;
  sh_w[t] = ri.w;
  __syncthreads();
  Seg re = Seg{shas[1], soff[2], soff[3]};
  if (t + 1 < kVjpScanThreads) re = seg_rl(Seg{sh_h[t + 1], sh_g[t + 1], sh_w[t + 1]}, re);
  // per tile: carry (exclusive, from the left) and cont (inclusive, from the right)
  Seg run = fe;
  double4 out[kVjpPer];
  for (int k = 0; k < kVjpPer; ++k) {
    out[k].x = run.g;
    out[k].y = run.w;
    run = seg_lr(run, tv[k]);
  }
  Seg back = re;
  for (int k = kVjpPer - 1; k >= 0; --k) {
    back = seg_rl(hv[k], back);
    out[k].z = back.g;
    out[k].w = back.w;
  }
  for (int k = 0; k < kVjpPer; ++k) {
    const int tt = b * kVjpBlock + kVjpPer * t + k;
    if (tt < ntile) cc[row * ntile + tt] = out[k];
  }
}

// Pass 3: each element's block sums from the two scans, seeded with its tile's carries.
// PACKED (rows of at most kVjpTile elements): a tile holds `rpt` whole rows, so no block crosses a
// tile and there are no carries; every row's first element starts a block whatever its flag says.
template <typename T, bool PACKED = false>
__global__ __launch_bounds__(kVjpThreads, 4) void k_vjp_apply(const T* __restrict__ g, const T* __restrict__ y,
                                                           const T* __restrict__ w, const T* __restrict__ z,
                                                           const uint8_t* __restrict__ bs,
                                                           const double4* __restrict__ cc, T* __restrict__ gy,
                                                           T* __restrict__ gw, int64_t n, int ntile,
                                                           int64_t batch = 1, int rpt = 1) {
  __shared__ Seg sh[2 * kVjpThreads / kWave];
  const int64_t tid = blockIdx.x;
  int64_t off;
  int len;
  int tt = 0;
  if constexpr (PACKED) {
    const int64_t r0 = tid * rpt;
    const int64_t nr = min((int64_t)rpt, batch - r0);
    off = r0 * n;
    len = (int)(nr * n);
  } else {
    const int64_t row = tid / ntile;
    tt = (int)(tid - row * ntile);
    off = row * n + (int64_t)tt * kVjpTile;
    const int64_t rem = n - (int64_t)tt * kVjpTile;
    len = rem < kVjpTile ? (int)rem : kVjpTile;
  }
  const int i0 = kVjpPer2 * threadIdx.x;
  const int c = min(max(len - i0, 0), kVjpPer2);
  // every load is issued here, the tile's carries included, before any of them is waited for
  const double4 zero4 = make_double4(0.0, 0.0, 0.0, 0.0);
  const double4 me = PACKED ? zero4 : cc[tid];
  const double4 nx = (PACKED || tt == ntile - 1) ? zero4 : cc[tid + 1];
  T gv[kVjpPer2], wv[kVjpPer2], yv[kVjpPer2], zv[kVjpPer2];
  vjp_load<T, true>(g, off + i0, c, gv, (T)0);
  if (w) vjp_load<T, true>(w, off + i0, c, wv, (T)0);
  vjp_load<T, true>(y, off + i0, c, yv, (T)0);
  vjp_load<T, true>(z, off + i0, c, zv, (T)0);
  int st[kVjpPer2 + 1];  // starts of this thread's elements and of the one after them
  if (kVjpPer2 == 8 && c == kVjpPer2 && ((uintptr_t)(bs + off + i0)) % 8 == 0) {
    const uint64_t b8 = *reinterpret_cast<const uint64_t*>(bs + off + i0);
#pragma unroll
    for (int k = 0; k < kVjpPer2; ++k) st[k] = ((b8 >> (8 * k)) & 0xffu) ? 1 : 0;
    st[kVjpPer2] = (i0 + kVjpPer2 < len) ? (bs[off + i0 + kVjpPer2] ? 1 : 0) : 0;
  } else {
#pragma unroll
    for (int k = 0; k <= kVjpPer2; ++k) st[k] = (k < c || (k == c && i0 + k < len)) ? (bs[off + i0 + k] ? 1 : 0) : 0;
  }
  if constexpr (PACKED) {
    // row starts (the tile starts at a row start)
    int rk = (i0 < len) ? (int)((int64_t)i0 % n) : 0;
#pragma unroll
    for (int k = 0; k <= kVjpPer2; ++k) {
      if (rk == 0 && (k < c || (k == c && i0 + k < len))) st[k] = 1;
      if (++rk == n) rk = 0;
    }
  }
  // forward fold (restart at starts) and backward fold (restart after block ends: the flag of
  // element k is the start of element k + 1)
  Seg f{0, 0.0, 0.0}, r{0, 0.0, 0.0};
#pragma unroll
  for (int k = 0; k < kVjpPer2; ++k) {
    if (k < c) f = seg_lr(f, Seg{st[k], (double)gv[k], w ? (double)wv[k] : 1.0});
  }
#pragma unroll
  for (int k = kVjpPer2 - 1; k >= 0; --k) {
    if (k < c) r = seg_rl(Seg{st[k + 1], (double)gv[k], w ? (double)wv[k] : 1.0}, r);
  }
  Seg fw, bw;
  vjp_wg_scans(f, r, Seg{0, me.x, me.y}, Seg{0, nx.z, nx.w}, sh, fw, bw);
  if (c == 0) return;
  double Fg[kVjpPer2], Fw[kVjpPer2];
  Seg run = fw;
#pragma unroll
  for (int k = 0; k < kVjpPer2; ++k) {
    if (k < c) {
      run = seg_lr(run, Seg{st[k], (double)gv[k], w ? (double)wv[k] : 1.0});
      Fg[k] = run.g;
      Fw[k] = run.w;
    }
  }
  T oy[kVjpPer2], ow[kVjpPer2];
  Seg back = bw;
#pragma unroll
  for (int k = kVjpPer2 - 1; k >= 0; --k) {
    oy[k] = (T)0;
    ow[k] = (T)0;
    if (k < c) {
      const double gd = (double)gv[k], wd = w ? (double)wv[k] : 1.0;
      back = seg_rl(Seg{st[k + 1], gd, wd}, back);
      const double G = Fg[k] + back.g - gd;
      const double Wt = Fw[k] + back.w - wd;
      const double q = G / Wt;
      oy[k] = (T)(wd * q);
      ow[k] = (T)(((double)yv[k] - (double)zv[k]) * q);
    }
  }
  constexpr int VN = Vec16<T>::N;
  const bool vec = c == kVjpPer2 && ((uintptr_t)(gy + off + i0)) % 16 == 0 &&
                   (!gw || ((uintptr_t)(gw + off + i0)) % 16 == 0);
  if (vec) {
#pragma unroll
    for (int k = 0; k < kVjpPer2 / VN; ++k) {
      store16_nt(gy + off + i0 + k * VN, &oy[k * VN]);
      if (gw) store16_nt(gw + off + i0 + k * VN, &ow[k * VN]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < kVjpPer2; ++k) {
      if (k < c) {
        gy[off + i0 + k] = oy[k];
        if (gw) gw[off + i0 + k] = ow[k];
      }
    }
  }
}

}  // namespace iso
