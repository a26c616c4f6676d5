// iso_row.h -- one row of up to 4096 elements per workgroup of 1024 threads (gfx950): rows of
// 2049 to 4096 elements, and shorter rows in batches too small to fill the chip otherwise.
//
// "Merge Hulls Without Copying Vertices: GPU Isotonic Regression":
//   Section 2      the fit is the slope sequence of the lower convex hull of the cumulative sum
//                  diagram (CSD) of (w, w y).
//   Section 3.1    each thread builds the hull of its own four elements' points (an inner point
//                  is a vertex iff it lies strictly below the segment of every pair around it).
//   Section 3.2 / Lemma 4.2   neighbouring hulls are merged pairwise, level by level, by their
//                  bridge: alpha the leftmost contact in the left hull, beta the rightmost in the
//                  right one, the vertices between them dropped.
//   Section 6 "Merge levels"  the bridge is searched by many threads at once rather than walked.
//   Section 6 "Coordinates" / "Predicates"   points are double-double pairs; a turn is decided on
//                  the hi parts when it clears an a-priori error bound, else from the pairs.
//
// A row that fits one workgroup's LDS is latency-bound whatever the kernel does, so this kernel
// spends threads on shortening the dependent chains:
//   - the whole diagram (up to 4097 points as pairs, 131 KB) sits in LDS, its sums scanned with
//     DPP row shifts;
//   - a thread's leaf hull has four points;
//   - a merge of two hulls by tpm threads gives each thread a few vertices a of the left hull,
//     finds by bisection the tangent point b(a) of the right hull seen from a, and keeps the a
//     whose neighbours both lie on or above the line a b(a) (the predecessor strictly above,
//     which makes a the leftmost contact); in a merge over several wavefronts whose pairs (a, b)
//     number at most tpm, each thread tests one pair instead, by the neighbours of both ends.  With exact turns exactly one
//     candidate passes; if rounding of a near-degenerate turn lets none or several pass, the
//     merge's threads all walk to the bridge instead, with the same result;
//   - a merge's threads are the ones that built its two nodes, so the levels whose merges fit in
//     one wavefront only wait for that wavefront.
// Hull vertex lists are kept compact, node k of level r at offset k m (m = 4 * 2^r points per
// node), without the node's last point (its end, always a vertex, implied), in one of two buffers
// that alternate by level.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "iso_geom.h"
#include "iso_merge.h"

namespace iso {

constexpr int kRowMax = 4096;  // elements of a row at most
// Elements per thread of the launched kernel (kRowMax / kRowP threads).  Measured per call on a
// 1 x 4096 fp64 weighted row: 4 elements 41.9 us, 8 elements 42.6 us, 16 elements 57.0 us (longer
// chains in fewer threads lose to more levels of parallel bridge searches); leaves of 8 or 16
// points chained by one thread of each group, with four elements per thread otherwise, took 48.2
// and 58.9 us against 39.9 us.
constexpr int kRowP = 4;

// LDS slot of point i with P points per thread: residue-major, so a thread's consecutive points
// are a column (kRowMax / P + 1 slots) apart and a wavefront's threads touch consecutive slots.
template <int P>
__device__ __forceinline__ int row_slot(int i) { return (i & (P - 1)) * (kRowMax / P + 1) + i / P; }

// A double moved by a DPP control; a lane whose source the control does not reach reads 0.
template <int CTRL>
__device__ __forceinline__ double dpp0(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(b & 0xffffffffll), CTRL, 0xf, 0xf, true);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, 0xf, 0xf, true);
  return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}
template <int CTRL>
__device__ __forceinline__ DD dpp0(DD a) { return DD{dpp0<CTRL>(a.hi), dpp0<CTRL>(a.lo)}; }

// lane l's value (l uniform over the wavefront)
__device__ __forceinline__ double lane_value(double v, int l) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffffll), l);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
  return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}
__device__ __forceinline__ DD lane_value(DD a, int l) { return DD{lane_value(a.hi, l), lane_value(a.lo, l)}; }

// Inclusive scans within each row of 16 lanes by DPP row shifts (1, 2, 4, 8): pairs summed with
// dd_add, the earlier part first, and plain doubles.
__device__ __forceinline__ DD row_scan(DD a) {
  a = dd_add(dpp0<0x111>(a), a);
  a = dd_add(dpp0<0x112>(a), a);
  a = dd_add(dpp0<0x114>(a), a);
  a = dd_add(dpp0<0x118>(a), a);
  return a;
}
__device__ __forceinline__ double row_scan(double a) {
  a += dpp0<0x111>(a);
  a += dpp0<0x112>(a);
  a += dpp0<0x114>(a);
  a += dpp0<0x118>(a);
  return a;
}

// Inclusive scan over the wavefront: rows of 16, then the earlier rows' totals (lanes 15, 31, 47).
__device__ __forceinline__ DD wave_scan(DD a, int row) {
  a = row_scan(a);
  const DD r0 = lane_value(a, 15), r1 = lane_value(a, 31), r2 = lane_value(a, 47);
  const DD p1 = r0, p2 = dd_add(r0, r1), p3 = dd_add(p2, r2);
  if (row > 0) a = dd_add(row == 1 ? p1 : row == 2 ? p2 : p3, a);
  return a;
}

template <typename T, bool W, bool D, int P>
__global__ __launch_bounds__(kRowMax / P) void k_row(const T* __restrict__ y, const T* __restrict__ w,
                                                      T* __restrict__ z, uint8_t* __restrict__ bstart,
                                                      uint32_t* __restrict__ rflags, int n, int walk) {
  constexpr bool EX = ExactProd<T, W>::value;
  constexpr int kRowPer = P;
  constexpr int kRowThreads = kRowMax / P;
  constexpr int kRowWaves = kRowThreads / kWave;
  constexpr int kRowSlots = P * (kRowThreads + 1);
  static_assert(P == 4 || P == 8 || P == 16, "4, 8 or 16 elements per thread");
  // points: weighted rows keep (x, y) hi parts together (one 16-byte read) and the lo parts
  // apart; unweighted rows keep y only (x is the index)
  __shared__ double2 sH[W ? kRowSlots : 1], sLo[W ? kRowSlots : 1];
  __shared__ double sYh[W ? 1 : kRowSlots], sYl[W ? 1 : kRowSlots];
  __shared__ uint16_t sL[2][kRowMax];          // vertex lists of the nodes of a level
  __shared__ uint16_t sC[2][kRowThreads];      // vertex counts: node k of level r at k 2^r
  __shared__ uint32_t sMin[kRowThreads];       // per merge group: level-tagged smallest (alpha, beta)
  __shared__ uint32_t sMax[kRowThreads];       // per merge group: level-tagged largest (alpha, beta)
  __shared__ double sW[16][5];                 // per wavefront: sums of the thread totals
  __shared__ uint32_t sFlag;

  const int t = threadIdx.x;
  const int wv = t >> 6, wl = t & (kWave - 1);
  const int64_t off = (int64_t)blockIdx.x * n;
  const int e0 = kRowPer * t;
  const int c = e0 >= n ? 0 : (n - e0 < kRowPer ? n - e0 : kRowPer);  // this thread's elements
  if (t == 0) sFlag = 0u;

  // ---- load: four consecutive elements per thread (16-byte vectors where aligned)
  T yv[kRowPer], wvv[kRowPer];
#pragma unroll
  for (int k = 0; k < kRowPer; ++k) {
    yv[k] = (T)0;
    wvv[k] = (T)1;
  }
  const bool vec = c == kRowPer && ((uintptr_t)(y + off + e0)) % 16 == 0 &&
                   (!W || ((uintptr_t)(w + off + e0)) % 16 == 0);
  if (vec) {
#pragma unroll
    for (int k = 0; k < kRowPer; k += Vec16<T>::N) {
      vload(y + off + e0 + k, &yv[k]);
      if (W) vload(w + off + e0 + k, &wvv[k]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < kRowPer; ++k) {
      if (k < c) {
        yv[k] = y[off + e0 + k];
        if (W) wvv[k] = w[off + e0 + k];
      }
    }
  }
  __syncthreads();  // sFlag cleared

  // ---- classify; the thread's increments (w, w y) as pairs, their sums, and the bound's sums
  double iw[kRowPer], ip[kRowPer], ie[kRowPer];
  uint32_t f = 0u;
  DD tx{0.0, 0.0}, ty{0.0, 0.0};
  double ta = 0.0;
#pragma unroll
  for (int k = 0; k < kRowPer; ++k) {
    double yd = yval<D>(yv[k]);
    double wd = W ? (double)wvv[k] : 1.0;
    if (k < c) {
      if (!isfinite(yd) || !isfinite(wd)) f |= ISO_ROW_NONFINITE_BIT;
      else if (!(wd > 0.0)) f |= ISO_ROW_BAD_WEIGHT_BIT;
      if (!isfinite(yd) || !isfinite(wd) || !(wd > 0.0)) {
        yd = 0.0;
        wd = 1.0;
      }
    } else {
      yd = 0.0;
      wd = 0.0;
    }
    const double p = wd * yd;
    iw[k] = wd;
    ip[k] = p;
    ie[k] = EX ? 0.0 : fma(wd, yd, -p);
    if (k < c) {
      if (W) acc(tx.hi, tx.lo, wd);
      acc_pe(ty.hi, ty.lo, p, ie[k]);
      ta += fabs(p);
    }
  }
  if (f) atomicOr(&sFlag, f);
  tx = two_sum(tx.hi, tx.lo);
  ty = two_sum(ty.hi, ty.lo);

  // ---- exclusive scan of the thread totals: in each wavefront (DPP row scans, then the rows'
  // totals), then over the wavefronts (a 16-lane scan of their totals in every wavefront)
  const int row = wl >> 4;
  const DD ix = W ? wave_scan(tx, row) : DD{0.0, 0.0};
  const DD iy = wave_scan(ty, row);
  double ia = row_scan(ta);
  ia = lane_value(ia, 15) + lane_value(ia, 31) + lane_value(ia, 47) + lane_value(ia, 63);
  const DD ex = dpp0<0x138>(ix), ey = dpp0<0x138>(iy);  // the previous lane's (wave_shr 1)
  if (wl == kWave - 1) {
    sW[wv][0] = ix.hi;
    sW[wv][1] = ix.lo;
    sW[wv][2] = iy.hi;
    sW[wv][3] = iy.lo;
    sW[wv][4] = ia;
  }
  __syncthreads();
  DD px{0.0, 0.0}, py{0.0, 0.0};
  double xr, ar;
  {
    const int v = wl & 15;
    const bool on = v < kRowWaves;
    const DD qx = W ? row_scan(on ? DD{sW[v][0], sW[v][1]} : DD{0.0, 0.0}) : DD{0.0, 0.0};
    const DD qy = row_scan(on ? DD{sW[v][2], sW[v][3]} : DD{0.0, 0.0});
    ar = row_scan(on ? sW[v][4] : 0.0);
    xr = lane_value(qx.hi, 15);
    ar = lane_value(ar, 15);
    const int src = __builtin_amdgcn_readfirstlane(wv > 0 ? wv - 1 : 0);
    if (wv > 0) {
      px = lane_value(qx, src);
      py = lane_value(qy, src);
    }
  }
  DD sx0 = px, sy0 = py;
  if (wl != 0) {
    sx0 = dd_add(px, ex);
    sy0 = dd_add(py, ey);
  }
  const double E = ((W ? xr : (double)n) * 0x1p-47) * ar;  // the row's turn bound

  // ---- points e0 .. e0 + c as pairs (the row's end point n written by the thread of its last
  // element), at their residue-major slots.
  {
    DD lx{0.0, 0.0}, ly{0.0, 0.0};
#pragma unroll
    for (int k = 0; k <= kRowPer; ++k) {
      if (k < c || (k == c && c > 0 && e0 + c == n)) {
        const int i = row_slot<P>(e0 + k);
        const DD Y = dd_add(sy0, ly);
        if constexpr (W) {
          const DD X = dd_add(sx0, lx);
          sH[i] = make_double2(X.hi, Y.hi);
          sLo[i] = make_double2(X.lo, Y.lo);
        } else {
          sYh[i] = Y.hi;
          sYl[i] = Y.lo;
        }
        if (k < kRowPer) {
          if (W) acc(lx.hi, lx.lo, iw[k]);
          acc_pe(ly.hi, ly.lo, ip[k], ie[k]);
        }
      }
    }
  }
  // the level-tagged bridge slots start empty
  sMin[t] = 0xffffffffu;
  sMax[t] = 0u;
  __syncthreads();

  // point i of the diagram (hi parts, and as a pair); x of an unweighted point is its index
  auto hp = [&](int i) -> double2 {
    const int u = row_slot<P>(i);
    if constexpr (W) return sH[u];
    else return make_double2((double)i, sYh[u]);
  };
  auto Q = [&](int i) -> PD {
    const int u = row_slot<P>(i);
    if constexpr (W) {
      const double2 h = sH[u], l = sLo[u];
      return PD{DD{h.x, l.x}, DD{h.y, l.y}};
    } else {
      return PD{DD{(double)i, 0.0}, DD{sYh[u], sYl[u]}};
    }
  };
  // strict left turn (i, j, k): the fast turn when it clears the bound, else the pairs' turn
  auto left3 = [&](int i, double ix_, double iy_, int j, double jx, double jy, int k, double kx,
                   double ky) -> bool {
    const double tt = turn_hi(ix_, iy_, jx, jy, kx, ky);
    if (fabs(tt) > E) return tt > 0.0;
    return turn_dd(Q(i), Q(j), Q(k)).hi > 0.0;
  };
  auto left = [&](int i, int j, int k) -> bool {
    const double2 pi = hp(i), pj = hp(j), pk = hp(k);
    return left3(i, pi.x, pi.y, j, pj.x, pj.y, k, pk.x, pk.y);
  };

  // ---- leaves: the hull of points e0 .. e0 + c, kept as the list of its vertices before e0 + c.
  // With four points, point e0 + k (0 < k < c) is a vertex iff it lies strictly below the segment
  // of every pair of points on either side of it (ten independent tests); with more, the
  // monotone chain.
  if (c > 0) {
    bool vtx[kRowPer];
    if constexpr (P == 4) {
      double lxv[kRowPer + 1], lyv[kRowPer + 1];
#pragma unroll
      for (int k = 0; k <= kRowPer; ++k) {
        lxv[k] = 0.0;
        lyv[k] = 0.0;
        if (k <= c) {
          const double2 h = hp(e0 + k);
          lxv[k] = h.x;
          lyv[k] = h.y;
        }
      }
#pragma unroll
      for (int k = 0; k < kRowPer; ++k) vtx[k] = k < c;
#pragma unroll
      for (int k = 1; k < kRowPer; ++k) {
#pragma unroll
        for (int a = 0; a < k; ++a) {
#pragma unroll
          for (int b = k + 1; b <= kRowPer; ++b) {
            if (b <= c && vtx[k] &&
                !left3(e0 + a, lxv[a], lyv[a], e0 + k, lxv[k], lyv[k], e0 + b, lxv[b], lyv[b]))
              vtx[k] = false;
          }
        }
      }
    } else {
      auto Pt = [&](int k, double& xx, double& yy) {
        const double2 h = hp(e0 + k);
        xx = h.x;
        yy = h.y;
      };
      auto Pq = [&](int k) -> PD { return Q(e0 + k); };
      const uint64_t mk = lane_chain(c, Pt, Pq, E);
#pragma unroll
      for (int k = 0; k < kRowPer; ++k) vtx[k] = k < c && ((mk >> k) & 1ull);
    }
    int q = 0;
#pragma unroll
    for (int k = 0; k < kRowPer; ++k)
      if (vtx[k]) sL[0][e0 + q++] = (uint16_t)(e0 + k);
    sC[0][t] = (uint16_t)q;
  }
  wave_sync();

  // ---- merge levels.  At level r a merge of nodes 2j and 2j + 1 (m points each) is done by the
  // tpm = 2^(r+1) threads j tpm .. (j + 1) tpm - 1, the threads that built those nodes, so while
  // tpm <= 64 a level only waits for its own wavefront.  A candidate that passes records
  // (alpha, beta) in the merge's two slots (index j tpm, used only by this thread group at every
  // level) with atomicMin and atomicMax on keys tagged by the level: the bridge is unique when
  // both slots hold this level's tag and the same (alpha, beta).  Node k's vertex count is kept at
  // index k 2^r, its first leaf, so that it too is only touched by the threads of its subtree.
  int nodes = (n + kRowPer - 1) / kRowPer;
  int m = kRowPer;  // points per node
  int cur = 0;
  for (int r = 0; nodes > 1; ++r) {
    const int merges = nodes >> 1;
    const int tpm = 2 << r;
    const int j = t >> (r + 1), q = t & (tpm - 1);
    const int slot = j * tpm;
    const uint16_t* LA = &sL[cur][2 * j * m];
    const uint16_t* LB = LA + m;
    int cA = 0, cB = 0, s = 0, e = 0;
    bool convex = true;
    if (j < merges) {
      cA = sC[cur][(2 * j) << r];
      cB = sC[cur][(2 * j + 1) << r];
      s = (2 * j + 1) * m;
      e = min((2 * j + 2) * m, n);
      // A' = LA[0..cA) + s, B' = LB[0..cB) + e, LB[0] = s
      const int b1 = cB > 1 ? LB[1] : e;
      convex = left(LA[cA - 1], s, b1);  // the union is convex at s: alpha = s, beta = b1
    }
    auto Ai = [&](int i) -> int { return i < cA ? (int)LA[i] : s; };
    auto Bk = [&](int k) -> int { return k < cB ? (int)LB[k] : e; };
    int al = cA, be = 1;
    const int npair = (cA + 1) * cB;  // candidate bridges (alpha, beta): alpha in A', beta in B' \ {s}
    const bool search = !convex && !walk;  // walk != 0: every bridge by the walk (testing)
    if (search && tpm > kWave && npair <= tpm) {
      // few enough pairs for one each: the pair (i, k) is the bridge iff A'[i]'s predecessor lies
      // strictly above the line A'[i] B'[k] and its successor on or above it, and B'[k]'s
      // successor strictly above and predecessor on or above (four independent turns).  Only for
      // merges over several wavefronts: below that the hulls are small, a bisection takes a step
      // or two, and four turns per pair cost more (measured on the 4096 ramp: levels 0-5 +3.6 us,
      // levels 6-9 -1.7 us).
      if (q < npair) {
        const int i = q / cB, k = 1 + (q - (q / cB) * cB);
        const int a = Ai(i), b = Bk(k);
        const int ap = i > 0 ? Ai(i - 1) : a, an = i < cA ? Ai(i + 1) : a;
        const int bp = Bk(k - 1), bn = k < cB ? Bk(k + 1) : b;
        const double2 pa = hp(a), pb = hp(b), pap = hp(ap), pan = hp(an), pbp = hp(bp), pbn = hp(bn);
        const bool c1 = i == 0 || left3(ap, pap.x, pap.y, a, pa.x, pa.y, b, pb.x, pb.y);
        const bool c2 = i == cA || !left3(a, pa.x, pa.y, an, pan.x, pan.y, b, pb.x, pb.y);
        const bool c3 = k == cB || left3(a, pa.x, pa.y, b, pb.x, pb.y, bn, pbn.x, pbn.y);
        const bool c4 = k == 1 || !left3(a, pa.x, pa.y, bp, pbp.x, pbp.y, b, pb.x, pb.y);
        if (c1 && c2 && c3 && c4) {
          const uint32_t pay = (uint32_t)i << 13 | (uint32_t)k;
          atomicMin(&sMin[slot], (uint32_t)(14 - r) << 28 | pay);
          atomicMax(&sMax[slot], (uint32_t)(r + 1) << 28 | pay);
        }
      }
    } else if (search) {
      for (int i = q; i <= cA; i += tpm) {
        const int a = Ai(i);
        const double2 pa = hp(a);
        const double ax = pa.x, ay = pa.y;
        // b(a): the first k >= 1 with (a, B'[k], B'[k+1]) a strict left turn, else cB
        int lo = 1, hi = cB;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          const int bm = Bk(mid), bn = Bk(mid + 1);
          const double2 pm = hp(bm), pn = hp(bn);
          if (left3(a, ax, ay, bm, pm.x, pm.y, bn, pn.x, pn.y)) hi = mid;
          else lo = mid + 1;
        }
        const int b = Bk(lo);
        const double2 pb = hp(b);
        const double bx = pb.x, by = pb.y;
        bool ok = true;
        if (i > 0) {
          const int p = Ai(i - 1);
          const double2 pp = hp(p);
          ok = left3(p, pp.x, pp.y, a, ax, ay, b, bx, by);
        }
        if (ok && i < cA) {
          const int nx = Ai(i + 1);
          const double2 pn = hp(nx);
          ok = !left3(a, ax, ay, nx, pn.x, pn.y, b, bx, by);
        }
        if (ok) {
          const uint32_t pay = (uint32_t)i << 13 | (uint32_t)lo;
          atomicMin(&sMin[slot], (uint32_t)(14 - r) << 28 | pay);
          atomicMax(&sMax[slot], (uint32_t)(r + 1) << 28 | pay);
        }
      }
    }
    if (tpm <= kWave) wave_sync();
    else __syncthreads();
    const int nxt = cur ^ 1;
    if (j < merges) {
      if (!convex) {
        al = cA;
        be = 1;
        const uint32_t kmin = sMin[slot], kmax = sMax[slot];
        const uint32_t pmask = (1u << 28) - 1u;
        if (search && (kmin >> 28) == (uint32_t)(14 - r) && (kmax >> 28) == (uint32_t)(r + 1) &&
            (kmin & pmask) == (kmax & pmask)) {
          al = (int)((kmin & pmask) >> 13);
          be = (int)(kmin & 8191u);
        } else {
          // rounding let none or several candidates pass: every thread of the merge walks to
          // the bridge from s (Lemma 4.2), with the same result
          for (int pass = 0; pass <= cA + cB; ++pass) {
            bool moved = false;
            while (al > 0 && !left(Ai(al - 1), Ai(al), Bk(be))) {
              --al;
              moved = true;
            }
            while (be < cB && !left(Ai(al), Bk(be), Bk(be + 1))) {
              ++be;
              moved = true;
            }
            if (!moved) break;
          }
        }
      }
      // merged list at node j of the next level (same offset as A): A'[0..alpha], B'[beta..cB)
      uint16_t* out = &sL[nxt][2 * j * m];
      const int tot = al + 1 + cB - be;
      for (int k = q; k < tot; k += tpm) out[k] = (uint16_t)(k <= al ? Ai(k) : (int)LB[be + k - al - 1]);
      if (q == 0) sC[nxt][j << (r + 1)] = (uint16_t)tot;
    } else if (j == merges && (nodes & 1)) {
      // the last node has no partner: it moves up unchanged
      const int ln = nodes - 1;
      const int cl = sC[cur][ln << r];
      for (int k = q; k < cl; k += tpm) sL[nxt][ln * m + k] = sL[cur][ln * m + k];
      if (q == 0) sC[nxt][ln << r] = (uint16_t)cl;
    }
    cur = nxt;
    nodes = (nodes + 1) >> 1;
    m <<= 1;
    // the next level's thread groups span 2 tpm threads; the emit reads the root from all
    if (2 * tpm <= kWave && nodes > 1) wave_sync();
    else __syncthreads();
  }

  // ---- emit: element i gets the slope of the root hull's edge over it; an element whose two
  // points are both vertices is a block of its own and gets its y, the block's exact mean
  const uint32_t bad = sFlag;
  if (c > 0) {
    const uint16_t* V = sL[cur];
    const int cnt = sC[cur][0];
    int lo = 0, hi = cnt - 1;  // last vertex <= e0 (vertex 0 is point 0)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int)V[mid] <= e0) lo = mid;
      else hi = mid - 1;
    }
    int k = lo;
    int a = V[k];
    int b = k + 1 < cnt ? (int)V[k + 1] : n;
    double slope = slope_dd(Q(a), Q(b));
    T zo[kRowPer];
    uint8_t bo[kRowPer];
#pragma unroll
    for (int u = 0; u < kRowPer; ++u) {
      zo[u] = (T)0;
      bo[u] = 0;
      if (u < c) {
        const int i = e0 + u;
        if (b <= i) {
          ++k;
          a = b;
          b = k + 1 < cnt ? (int)V[k + 1] : n;
          slope = slope_dd(Q(a), Q(b));
        }
        const bool isv = a == i;
        zo[u] = bad ? (T)NAN : (isv && b == i + 1) ? yv[u] : (T)zval<D>(slope);
        bo[u] = (!bad && isv) ? 1 : 0;
      }
    }
    if (vec && ((uintptr_t)(z + off + e0)) % 16 == 0) {
#pragma unroll
      for (int u = 0; u < kRowPer; u += Vec16<T>::N) store16(z + off + e0 + u, &zo[u]);
    } else {
#pragma unroll
      for (int u = 0; u < kRowPer; ++u)
        if (u < c) z[off + e0 + u] = zo[u];
    }
    if (bstart) {
#pragma unroll
      for (int u = 0; u < kRowPer; ++u)
        if (u < c) bstart[off + e0 + u] = bo[u];
    }
  }
  if (t == 0 && rflags) rflags[blockIdx.x] = bad;
}

}  // namespace iso
