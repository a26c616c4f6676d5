// iso_geom.h -- geometry of the cumulative sum diagram (CSD) shared by the HIP kernels.
//
// Everything here is __host__ __device__ and free of launch or memory-space assumptions:
// points are read through accessor functors, so the kernels bind them to LDS or global memory.
//
// Source: "Merge Hulls Without Copying Vertices: GPU Isotonic Regression".
//   Section 2.1  the fit is the slope sequence of the lower hull of the CSD; a point on the
//                segment between its neighbours is not a vertex (turn == 0 means non-convex).
//   Section 3.1  lane hulls by the monotone chain with the stack held in a bit mask.
//   Section 3.2 / Lemma 4.2  two neighbouring hulls sharing their boundary point s merge along
//                a unique bridge; walking from s finds it (left end moves left while its turn
//                is not strictly left, right end moves right symmetrically).
//   Section 3.3 / Definition 4.3 / Theorem 4.4  segment lists: a node's hull is a sequence of
//                (chunk, first, last) ranges of chunk hulls, at most one per chunk; a merge
//                cuts one segment of each child and moves the right child's tail down.
//   Section 2.2 / 5.2  Overmars-van Leeuwen simultaneous bisection for the bridge of two
//                x-separated hulls.  The page's case analysis (its Appendix A) did not survive,
//                so the cases below are derived here from the slopes; see bridge_search().
//   Section 6 "Coordinates" / "Predicates"  every coordinate is a pair (hi, lo) whose sum is
//                the coordinate: running sums carry the exact rounding error of each addition
//                (and of each product w*y) in lo, lane and chunk starts are double-double.  A turn
//                is first evaluated on the hi parts; when it falls inside an a-priori bound on
//                the error of that evaluation, it is recomputed from the pairs in double-double
//                arithmetic.  Slopes are formed from double-double differences.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define ISO_HD __host__ __device__ __forceinline__

namespace iso {

constexpr int kWave = 64;                    // lanes of a wavefront
constexpr int kLanePts = 32;                 // elements per lane of a packed short-row tile
constexpr int kShortMax = 2 * kWave * kLanePts;  // rows of at most this many go to the short-row kernel
constexpr int kSub = 256;                    // points per lane of a long-row chunk
constexpr int kChunk = kWave * kSub;         // elements per chunk of a long row (one wavefront)
constexpr int kCk = 32;                      // spacing of a lane's running-sum checkpoints
constexpr int kLaneW = kSub / kCk;           // mask words (and checkpoints) per lane
constexpr int kSubW = kLaneW + 1;            // mask words of a lane's points 0..256
constexpr int kListCap = 256;                // chunks with at most this many hull vertices keep a list
constexpr int kMaskW = kChunk / 32 + 1;      // mask words of a chunk (points 0..16384)
constexpr int kZT = 8;                       // elements per z-tile mark of the chunk pass (32 per lane)
constexpr int kVjpTile = kWave * 32;         // elements per backward tile (256 threads, 8 each)

// Per-row input flags (same values as ISO_ROW_NONFINITE / ISO_ROW_BAD_WEIGHT of iso.h).
constexpr uint32_t ISO_ROW_NONFINITE_BIT = 1u;
constexpr uint32_t ISO_ROW_BAD_WEIGHT_BIT = 2u;

// ------------------------------------------------------------------ arithmetic

// (ax, ay) x (bx, by) with one rounded product.
ISO_HD double cross2(double ax, double ay, double bx, double by) { return fma(ax, by, -(ay * bx)); }

// An input value as the diagram uses it.  The decreasing fit (z_0 >= ... >= z_{n-1}) is the
// negated increasing fit of -y; negation is exact and rounding to nearest is symmetric, so with D
// every sum, turn and slope is the exact mirror of the increasing fit's of -y.
template <bool D, typename T>
ISO_HD double yval(T v) {
  return D ? -(double)v : (double)v;
}
// A fitted slope as the caller receives it.
template <bool D>
ISO_HD double zval(double s) {
  return D ? -s : s;
}

struct DD {
  double hi, lo;
};

ISO_HD DD two_sum(double a, double b) {
  double s = a + b;
  double bb = s - a;
  double e = (a - (s - bb)) + (b - bb);
  return {s, e};
}

ISO_HD DD quick_two_sum(double a, double b) {
  double s = a + b;
  double e = b - (s - a);
  return {s, e};
}

// Double-double addition (accurate to about 2^-104 relative).
ISO_HD DD dd_add(DD a, DD b) {
  DD s = two_sum(a.hi, b.hi);
  DD t = two_sum(a.lo, b.lo);
  double e = s.lo + t.hi;
  s = quick_two_sum(s.hi, e);
  e = s.lo + t.lo;
  return quick_two_sum(s.hi, e);
}

ISO_HD DD two_prod(double a, double b) {
  const double p = a * b;
  return {p, fma(a, b, -p)};
}

ISO_HD DD dd_neg(DD a) { return {-a.hi, -a.lo}; }
ISO_HD DD dd_sub(DD a, DD b) { return dd_add(a, dd_neg(b)); }

ISO_HD DD dd_mul(DD a, DD b) {
  DD p = two_prod(a.hi, b.hi);
  const double c = a.hi * b.lo + a.lo * b.hi;
  return quick_two_sum(p.hi, p.lo + c);
}

// Running sums.  acc adds v to the pair (hi, lo): hi becomes the rounded sum, as a plain fp64
// running sum would, and the exact error of that addition goes to lo.  acc_pe adds a product p
// whose own rounding error pe is known (zero when the product is exact).  After k additions
// |lo| <= k u max|partial sum| (+ u sum|p| for inexact products), u = 2^-53.
ISO_HD void acc_pe(double& hi, double& lo, double v, double pe) {
  const double s = hi + v;
  const double bb = s - hi;
  const double e = (hi - (s - bb)) + (v - bb);
  lo += e + pe;
  hi = s;
}
ISO_HD void acc(double& hi, double& lo, double v) {
  const double s = hi + v;
  const double bb = s - hi;
  const double e = (hi - (s - bb)) + (v - bb);
  lo += e;
  hi = s;
}

// The increment w*y of one element.  For fp32 inputs and for unit weights the fp64 product is
// exact; otherwise its rounding error is added to lo.
template <bool EXACT>
ISO_HD void acc_prod(double& hi, double& lo, double w, double y) {
  const double p = w * y;
  if constexpr (EXACT) acc(hi, lo, p);
  else acc_pe(hi, lo, p, fma(w, y, -p));
}
template <typename T, bool W>
struct ExactProd {
  static constexpr bool value = !W || sizeof(T) == 4;
};

// A point of the diagram as a pair of double-double coordinates.
struct PD {
  DD x, y;
};

// turn(a, b, c) = (b - a) x (c - a) in double-double arithmetic (relative error a few u^2 of
// the two products); its sign decides the predicate when the fast evaluation cannot.
ISO_HD DD turn_dd(const PD& a, const PD& b, const PD& c) {
  const DD dx1 = dd_sub(b.x, a.x), dy1 = dd_sub(b.y, a.y);
  const DD dx2 = dd_sub(c.x, a.x), dy2 = dd_sub(c.y, a.y);
  return dd_sub(dd_mul(dx1, dy2), dd_mul(dy1, dx2));
}

// dy / dx for double-double differences, rounded once (within about one ulp of the quotient of
// the pairs): the quotient of the hi parts corrected by its remainder.
ISO_HD double dd_quot(DD dy, DD dx) {
  const double q = dy.hi / dx.hi;
  const DD p = two_prod(q, dx.hi);
  const double r = (((dy.hi - p.hi) - p.lo) + dy.lo) - q * dx.lo;
  return q + r / dx.hi;
}

ISO_HD double slope_dd(const PD& a, const PD& b) { return dd_quot(dd_sub(b.y, a.y), dd_sub(b.x, a.x)); }

// Device-wide counts of rarely taken branches, read and reset by iso_prof_counters: [0] merges of
// the merge levels that fell back on the Overmars-van Leeuwen bisection, [1] bisections that
// rounding defeated (finished by single steps), [2] chunks processed by the exact chunk pass,
// [3] merges that walked in memory windows.  Each is one atomic add by one lane, on its path only.
__device__ unsigned long long g_branch_counts[4];

// A little above u = 2^-53: the error of a rounded operation relative to its rounded result.
constexpr double kU = 0x1.0001p-53;

// Fast turn of three points given by their hi parts, for a predicate filter: t = turn(a, b, c)
// with one rounded product.
ISO_HD double turn_hi(double ax, double ay, double bx, double by, double cx, double cy) {
  return cross2(bx - ax, by - ay, cx - ax, cy - ay);
}

// ------------------------------------------------------------------ lane hull

// Monotone chain over the points 0..c of one lane (c <= 32), read through P(k, &x, &y) (hi
// parts) and Q(k) (the point as a PD).  Returns the hull as a bit mask (bit k set iff point k is
// a vertex).  A point is popped when the turn (under, top, next) is <= 0, so collinear middle
// points are dropped; a fast turn within E of zero is decided by turn_dd.  Every iteration
// either pops or pushes, and exactly one point load is issued per iteration.
template <class PtFn, class PdFn>
ISO_HD uint64_t lane_chain(int c, PtFn P, PdFn Q, double E) {
  if (c <= 0) return 0;
  if (c == 1) return 3ull;
  uint64_t mask = 3ull;
  int top = 1, und = 0, k = 2;
  double ux, uy, tx, ty, kx, ky;
  P(0, ux, uy);
  P(1, tx, ty);
  P(2, kx, ky);
  // <= 2c iterations: each point is pushed once and popped at most once.
  for (int it = 0; it < 2 * kLanePts + 2 && k <= c; ++it) {
    double t = turn_hi(ux, uy, tx, ty, kx, ky);
    if (!(fabs(t) > E)) t = turn_dd(Q(und), Q(top), Q(k)).hi;
    bool pop = (top != 0) && (t <= 0.0);
    int load_idx;
    if (pop) {
      mask &= ~(1ull << top);
      top = und;
      tx = ux;
      ty = uy;
      uint64_t below = mask & ((1ull << und) - 1ull);
      und = below ? 63 - __builtin_clzll(below) : 0;
      load_idx = und;
    } else {
      mask |= 1ull << k;
      und = top;
      ux = tx;
      uy = ty;
      top = k;
      tx = kx;
      ty = ky;
      ++k;
      load_idx = k <= c ? k : c;
    }
    double lx, ly;
    P(load_idx, lx, ly);
    if (pop) {
      ux = lx;
      uy = ly;
    } else {
      kx = lx;
      ky = ly;
    }
  }
  return mask;
}

// ------------------------------------------------------------------ bit-mask neighbours

// Vertex sets of a tile are bit masks: point k is word k >> 5, bit k & 31.
// Largest set bit strictly below k (one exists: the caller's node start is a vertex).
ISO_HD int mask_pred(const uint32_t* M, int k) {
  int u = k >> 5;
  uint32_t m = M[u] & ((1u << (k & 31)) - 1u);
  while (m == 0) m = M[--u];
  return (u << 5) + 31 - __builtin_clz(m);
}

// Smallest set bit strictly above k (one exists: the caller's node end is a vertex).
ISO_HD int mask_succ(const uint32_t* M, int k) {
  int u = k >> 5;
  int b = k & 31;
  uint32_t m = (b == 31) ? 0u : (M[u] & ~((2u << b) - 1u));
  while (m == 0) m = M[++u];
  return (u << 5) + __builtin_ctz(m);
}

// Clears the bits strictly between a and b (a < b).  Words holding no bit of (a, b) are not
// written, so merges of disjoint nodes never write the same word.
ISO_HD void mask_clear_between(uint32_t* M, int a, int b) {
  int ua = a >> 5, ub = b >> 5;
  for (int u = ua; u <= ub; ++u) {
    int lo = (u == ua) ? (a & 31) + 1 : 0;    // first bit to clear
    int hi = (u == ub) ? (b & 31) : 32;       // one past the last
    if (lo >= hi) continue;
    uint32_t keep_lo = lo >= 32 ? 0xffffffffu : ((1u << lo) - 1u);
    uint32_t keep_hi = hi >= 32 ? 0u : ~((1u << hi) - 1u);
    M[u] &= (keep_lo | keep_hi);
  }
}

// Merge of two neighbouring nodes of one tile by walking (Lemma 4.2): node A spans points
// [a0, s], node B spans [s, b1]; vertices are set bits of M, coordinates come from P (hi parts)
// and Q (pairs), with fast turns within E of zero decided by turn_dd.
// The bridge (alpha, beta) is found with alpha the leftmost contact in A (s included) and beta
// the rightmost contact in B \ {s}; the bits strictly between them are cleared.
template <class PtFn, class PdFn>
ISO_HD void tile_walk_merge(uint32_t* M, int a0, int s, int b1, PtFn P, PdFn Q, double E) {
  int al = s;
  int be = mask_succ(M, s);
  double ax, ay, bx, by;
  P(al, ax, ay);
  P(be, bx, by);
  auto left = [&](int i, double ix, double iy, int j, double jx, double jy, int k, double kx, double ky) {
    const double t = turn_hi(ix, iy, jx, jy, kx, ky);
    if (fabs(t) > E) return t > 0.0;
    return turn_dd(Q(i), Q(j), Q(k)).hi > 0.0;
  };
  // Each move removes a vertex of A or B, so the total number of moves is below b1 - a0.
  for (int pass = 0; pass <= b1 - a0; ++pass) {
    bool moved = false;
    while (al != a0) {
      int p = mask_pred(M, al);
      double px, py;
      P(p, px, py);
      if (!left(p, px, py, al, ax, ay, be, bx, by)) {
        al = p;
        ax = px;
        ay = py;
        moved = true;
      } else {
        break;
      }
    }
    while (be != b1) {
      int q = mask_succ(M, be);
      double qx, qy;
      P(q, qx, qy);
      if (!left(al, ax, ay, be, bx, by, q, qx, qy)) {
        be = q;
        bx = qx;
        by = qy;
        moved = true;
      } else {
        break;
      }
    }
    if (!moved) break;
  }
  mask_clear_between(M, al, be);
}

// ------------------------------------------------------------------ segment lists

// A point in row coordinates: the chunk's double-double start (sxh, syh: hi parts) plus the
// point's chunk-relative coordinates (x, y: hi parts), with the start's lo part and the local
// lo part added into sxl, syl.  The represented coordinate is sxh + sxl + x (and likewise y):
// folding the two lo parts costs a rounding of u |sxl|, far below the pairs' own accuracy.
struct GPt {
  double x, y;
  double sxh, sxl, syh, syl;
};

// q - p with the coordinate hierarchy, on doubles: the start difference first (exact for nearby
// chunks by Sterbenz's lemma; zero within one chunk), then the local difference.  ex, ey bound
// the error against the represented difference: every rounded operation contributes at most kU
// times its result.
ISO_HD void gdiff(const GPt& p, const GPt& q, double& dx, double& dy, double& ex, double& ey) {
  const double ax = q.sxh - p.sxh, bx = q.sxl - p.sxl, cx = ax + bx, lx = q.x - p.x;
  dx = cx + lx;
  ex = kU * (fabs(ax) + fabs(bx) + fabs(cx) + fabs(lx) + fabs(dx));
  const double ay = q.syh - p.syh, by = q.syl - p.syl, cy = ay + by, ly = q.y - p.y;
  dy = cy + ly;
  ey = kU * (fabs(ay) + fabs(by) + fabs(cy) + fabs(ly) + fabs(dy));
}

// q - p of the represented coordinates in double-double arithmetic.
ISO_HD DD gdx_dd(const GPt& p, const GPt& q) {
  return dd_add(dd_sub(DD{q.sxh, q.sxl}, DD{p.sxh, p.sxl}), two_sum(q.x, -p.x));
}
ISO_HD DD gdy_dd(const GPt& p, const GPt& q) {
  return dd_add(dd_sub(DD{q.syh, q.syl}, DD{p.syh, p.syl}), two_sum(q.y, -p.y));
}

ISO_HD DD gturn_dd(const GPt& a, const GPt& b, const GPt& c) {
  const DD dx1 = gdx_dd(a, b), dy1 = gdy_dd(a, b), dx2 = gdx_dd(a, c), dy2 = gdy_dd(a, c);
  return dd_sub(dd_mul(dx1, dy2), dd_mul(dy1, dx2));
}

// turn(a, b, c) > 0 (a strict left turn): the fast turn when it exceeds its error bound, else the
// sign of the double-double turn.  With |DX - dx| <= ex and so on, the fast turn
// fma(dx1, dy2, -fl(dy1 dx2)) is within
//   ex1 (|dy2| + ey2) + ey2 |dx1| + ex2 (|dy1| + ey1) + ey1 |dx2| + u (|dy1 dx2| + |t|)
// of the turn of the represented points; the bound itself is evaluated with a margin for its
// own rounding.
// The rare second evaluation (inline: a call would pin the live registers of every call site).
__device__ __forceinline__ bool gleft_slow(const GPt& a, const GPt& b, const GPt& c) { return gturn_dd(a, b, c).hi > 0.0; }

__device__ __forceinline__ bool gleft(const GPt& a, const GPt& b, const GPt& c) {
  double dx1, dy1, dx2, dy2, ex1, ey1, ex2, ey2;
  gdiff(a, b, dx1, dy1, ex1, ey1);
  gdiff(a, c, dx2, dy2, ex2, ey2);
  const double p2 = dy1 * dx2;
  const double t = fma(dx1, dy2, -p2);
  double E = ex1 * (fabs(dy2) + ey2) + ey2 * fabs(dx1) + ex2 * (fabs(dy1) + ey1) + ey1 * fabs(dx2) +
             kU * (fabs(p2) + fabs(t));
  E = E * 1.001 + 0x1p-1000;
  if (fabs(t) > E) return t > 0.0;
  return gleft_slow(a, b, c);
}

// Slope of the edge from a to b, from double-double differences.
ISO_HD double gslope(const GPt& a, const GPt& b) { return dd_quot(gdy_dd(a, b), gdx_dd(a, b)); }

// Segment descriptor: x = chunk index within the row, y = first vertex position, z = last
// vertex position (positions count the chunk hull's vertices from 0), w = the chunk hull's
// storage form (bits 0-1: 0 list, 1 dense, 2 dense form of an all-vertex chunk) and vertex count
// (bits 2 and up).
using Desc = int4;

ISO_HD int desc_w(int form, int nverts) { return form | (nverts << 2); }
ISO_HD int desc_form(const Desc& d) { return d.w & 3; }
ISO_HD int desc_nverts(const Desc& d) { return d.w >> 2; }

// ------------------------------------------------------------------ chunk hull storage
// A chunk's hull is stored in one of two forms:
//   list   the vertices' chunk-relative coordinate pairs and chunk point indices, in order (hulls
//          of at most kListCap vertices);
//   dense  the vertex bit mask of the chunk's points 0..16384, the number of set bits before
//          each word, the lane starts and every lane's running sums at each 32nd point, all as
//          pairs.  A vertex's pairs are recomputed from these and the inputs with the same fp64
//          operations in the same order as the chunk pass, so they are bitwise its values.
// Dense chunks are the ones whose points nearly all survive; storing them as lists would move
// about 34 bytes per element, while the dense form takes under two.
//
// Chunk-relative point k of lane l (k = 256 l + q) is the double-double sum of the lane's start
// S_l and the lane-relative running sum a(q) (accumulated with acc from the checkpoint below q);
// a lane's end point is the next lane's start, the chunk's end point its total.
template <typename T, bool W, bool D>
struct VertexStore {
  static constexpr bool EX = ExactProd<T, W>::value;
  Desc* desc;             // [G] descriptor slots
  int* nseg;              // [G] length of the list of the node starting at this slot
  const int* nverts;      // [G] vertex count of each chunk hull
  const uint8_t* dense;   // [G] 0 list form, 1 dense form, 2 dense form of an all-vertex chunk
  const double* lx;       // [G * kListCap] list form (pairs)
  const double* ly;
  const uint16_t* lk;
  const uint32_t* mask;   // [G * kMaskW] dense form
  const uint16_t* mcnt;   // [G * kMaskW]
  const double* lsx;      // [G * kWave]  lane starts (weighted only: x), pairs
  const double* lsy;
  const double* ckx;      // [G * kWave * kLaneW] lane-relative running sums (weighted only: x)
  const double* cky;
  const double2* tot;     // [G] chunk end point (W, S), hi and lo parts
  const double4* start;   // [G] chunk start {x hi, x lo, y hi, y lo}
  const double4* bnd;     // [G] dense form: vertices 1 and V - 2 {x1, y1, x2, y2}, hi and lo parts
  const int2* bndk;       // [G] their point indices
  const T* y;
  const T* w;
  int64_t n;              // row length
  int m;                  // chunks per row
  int64_t G;              // chunks of the call: each lo array follows its hi array, G chunks on

  ISO_HD const double* lxl() const { return lx + G * kListCap; }
  ISO_HD const double* lyl() const { return ly + G * kListCap; }
  ISO_HD const double* lsxl() const { return lsx + G * kWave; }
  ISO_HD const double* lsyl() const { return lsy + G * kWave; }
  ISO_HD const double* ckxl() const { return ckx + G * (kWave * kLaneW); }
  ISO_HD const double* ckyl() const { return cky + G * (kWave * kLaneW); }
  ISO_HD const double2* totl() const { return tot + G; }
  ISO_HD const double4* bndl() const { return bnd + G; }

  ISO_HD bool is_list(int64_t g) const { return dense[g] == 0; }

  // Lane start S_l and lane-relative running sum a at point k (0 <= k < len) of dense chunk j:
  // point k is S_l + a (for unit weights x is k itself), and adding elements k, k + 1, ... to a
  // with acc gives the points after k up to the next multiple of 32.
  ISO_HD void dense_state(int64_t row, int j, int k, DD& sx, DD& sy, DD& ax, DD& ay) const {
    const int64_t g = row * m + j;
    const int l = k / kSub, q = k % kSub;
    sx = W ? DD{lsx[g * kWave + l], lsxl()[g * kWave + l]} : DD{(double)(kSub * l), 0.0};
    sy = DD{lsy[g * kWave + l], lsyl()[g * kWave + l]};
    ax = DD{0.0, 0.0};
    ay = DD{0.0, 0.0};
    if (q == 0) return;
    const int jj = q / kCk;
    const int64_t cb = g * (int64_t)(kWave * kLaneW) + jj * kWave + l;
    if (W) ax = DD{ckx[cb], ckxl()[cb]};
    ay = DD{cky[cb], ckyl()[cb]};
    const int64_t e0 = row * n + (int64_t)j * kChunk + (int64_t)l * kSub;
    for (int e = kCk * jj; e < q; ++e) {
      double wd = W ? (double)w[e0 + e] : 1.0;
      double yd = yval<D>(y[e0 + e]);
      if (!isfinite(yd) || !isfinite(wd) || !(wd > 0.0)) {
        yd = 0.0;
        wd = 1.0;
      }
      if (W) acc(ax.hi, ax.lo, wd);
      acc_prod<EX>(ay.hi, ay.lo, wd, yd);
    }
  }

  // The point whose lane start is (sx, sy) and lane-relative running sum (ax, ay), chunk point k.
  ISO_HD static PD join(const DD& sx, const DD& sy, const DD& ax, const DD& ay, int k) {
    return PD{W ? dd_add(sx, ax) : DD{(double)k, 0.0}, dd_add(sy, ay)};
  }

  // Chunk-relative pairs of point k (0..len) of dense chunk j of `row`.
  ISO_HD PD dense_point(int64_t row, int j, int k) const {
    const int64_t g = row * m + j;
    const int64_t rem = n - (int64_t)j * kChunk;
    const int len = rem < kChunk ? (int)rem : kChunk;
    if (k == len) {
      const double2 t = tot[g], tl = totl()[g];
      return PD{DD{t.x, tl.x}, DD{t.y, tl.y}};
    }
    DD sx, sy, ax, ay;
    dense_state(row, j, k, sx, sy, ax, ay);
    if (k % kSub == 0) return PD{sx, sy};
    return join(sx, sy, ax, ay, k);
  }

  // Chunk-relative pairs and point index of vertex p of chunk j of `row`.
  ISO_HD PD local(int64_t row, int j, int p, int& k) const {
    const int64_t g = row * m + j;
    if (dense[g] == 0) {
      const int64_t idx = g * kListCap + p;
      k = lk[idx];
      return PD{DD{lx[idx], lxl()[idx]}, DD{ly[idx], lyl()[idx]}};
    }
    // the vertices the merges and ends touch most: the chunk's two ends and their neighbours
    const int V = nverts[g];
    if (p == 0) {
      k = 0;
      return PD{DD{0.0, 0.0}, DD{0.0, 0.0}};
    }
    if (p == V - 1) {
      const int64_t rem = n - (int64_t)j * kChunk;
      k = rem < kChunk ? (int)rem : kChunk;
      const double2 t = tot[g], tl = totl()[g];
      return PD{DD{t.x, tl.x}, DD{t.y, tl.y}};
    }
    if (p == 1 || p == V - 2) {
      const double4 b = bnd[g], bl = bndl()[g];
      const int2 bk = bndk[g];
      if (p == 1) {
        k = bk.x;
        return PD{DD{b.x, bl.x}, DD{b.y, bl.y}};
      }
      k = bk.y;
      return PD{DD{b.z, bl.z}, DD{b.w, bl.w}};
    }
    // select: the word holding the p-th set bit (the last word whose count of earlier set bits
    // is <= p), starting from where it would be if the bits were spread evenly, then the bit
    const uint16_t* mc = mcnt + g * kMaskW;
    int lo = (int)(((int64_t)p * (kMaskW - 1)) / (V > 0 ? V : 1));
    lo = lo < 0 ? 0 : (lo > kMaskW - 1 ? kMaskW - 1 : lo);
    while (lo > 0 && (int)mc[lo] > p) --lo;
    while (lo + 1 < kMaskW && (int)mc[lo + 1] <= p) ++lo;
    uint32_t word = mask[g * kMaskW + lo];
    for (int r = p - (int)mc[lo]; r > 0; --r) word &= word - 1u;
    k = lo * 32 + __builtin_ctz(word);
    return dense_point(row, j, k);
  }

  ISO_HD static GPt make_gpt(const PD& P, const double4& s) {
    GPt r;
    r.x = P.x.hi;
    r.y = P.y.hi;
    r.sxh = s.x;
    r.sxl = s.y + P.x.lo;
    r.syh = s.z;
    r.syl = s.w + P.y.lo;
    return r;
  }

  // pt() for a chunk known to be in list form (one round of independent loads).
  ISO_HD GPt pt_list(int64_t row, int j, int p) const {
    const int64_t g = row * m + j;
    const int64_t idx = g * kListCap + p;
    return make_gpt(PD{DD{lx[idx], lxl()[idx]}, DD{ly[idx], lyl()[idx]}}, start[g]);
  }

  // pt() of vertex p of the chunk of descriptor d, whose form and vertex count the descriptor
  // carries: list vertices and the dense form's cached ones need one round of loads.
  ISO_HD GPt pt_desc(int64_t row, const Desc& d, int p) const {
    const int form = desc_form(d), V = desc_nverts(d);
    if (form == 0) return pt_list(row, d.x, p);
    const int64_t g = row * m + d.x;
    if (p == 0 || p == V - 1 || p == 1 || p == V - 2) {
      PD P;
      if (p == 0) {
        P = PD{DD{0.0, 0.0}, DD{0.0, 0.0}};
      } else if (p == V - 1) {
        const double2 t = tot[g], tl = totl()[g];
        P = PD{DD{t.x, tl.x}, DD{t.y, tl.y}};
      } else {
        const double4 b = bnd[g], bl = bndl()[g];
        P = p == 1 ? PD{DD{b.x, bl.x}, DD{b.y, bl.y}} : PD{DD{b.z, bl.z}, DD{b.w, bl.w}};
      }
      return make_gpt(P, start[g]);
    }
    return pt(row, d.x, p);
  }

  ISO_HD GPt pt(int64_t row, int j, int p) const {
    int k;
    const PD P = local(row, j, p, k);
    return make_gpt(P, start[row * m + j]);
  }
};

struct VRef {
  int u;  // segment index within the node's list
  int p;  // vertex position within that segment's chunk hull
};

ISO_HD bool vref_eq(VRef a, VRef b) { return a.u == b.u && a.p == b.p; }
ISO_HD bool vref_le(VRef a, VRef b) { return a.u < b.u || (a.u == b.u && a.p <= b.p); }

// A node's segment list: descriptors d[0..n) in global memory, of row `row`.
struct NodeList {
  const Desc* d;
  int n;
  int64_t row;
};

template <class VS>
ISO_HD GPt load_v(const VS& S, const NodeList& L, VRef v) {
  const Desc d = L.d[v.u];
  return S.pt_desc(L.row, d, v.p);
}

ISO_HD VRef list_first(const NodeList& L) { return {0, L.d[0].y}; }
ISO_HD VRef list_last(const NodeList& L) { return {L.n - 1, L.d[L.n - 1].z}; }

ISO_HD VRef list_pred(const NodeList& L, VRef v) {
  if (v.p > L.d[v.u].y) return {v.u, v.p - 1};
  return {v.u - 1, L.d[v.u - 1].z};
}

ISO_HD VRef list_succ(const NodeList& L, VRef v) {
  if (v.p < L.d[v.u].z) return {v.u, v.p + 1};
  return {v.u + 1, L.d[v.u + 1].y};
}

// A vertex strictly inside [lo, hi] (or lo itself when the range has one or two vertices),
// splitting first at segment boundaries and then within one segment.
ISO_HD VRef list_mid(const NodeList& L, VRef lo, VRef hi) {
  if (lo.u == hi.u) return {lo.u, (lo.p + hi.p) >> 1};
  int um = (lo.u + hi.u + 1) >> 1;
  return {um, L.d[um].y};
}

// Overmars-van Leeuwen simultaneous bisection for the bridge of two x-separated lower hulls.
//
// A is the left hull (its last vertex s at abscissa x_s), B the right hull without s (every
// vertex right of x_s).  The bridge (alpha, beta) is the common tangent below both with alpha
// the leftmost and beta the rightmost contact.  With e_i the slope of A's edge leaving a_i,
// f_k the slope of B's edge leaving b_k and m the slope of a candidate pair (a_i, b_k):
//   A-case b: e_{i-1} >= m (pred(a_i) on or below the line a_i b_k)      => alpha < i
//   A-case a: e_i < m (succ(a_i) strictly below the line)
//   A-case c: otherwise (a_i is the tangent point of A seen from b_k)
//   B-case b: f_k <= m (succ(b_k) on or below the line)                   => beta > k
//   B-case a: f_{k-1} > m (pred(b_k) strictly below the line)
//   B-case c: otherwise
//   (a, c) => alpha > i;  (c, a) => beta < k;  (c, c) => (a_i, b_k) is the bridge;
//   (a, a) => the edge lines l_A through (a_i, a_{i+1}) and l_B through (b_{k-1}, b_k) cross at
//             some x_int: if l_B is on or above l_A at x_s (x_int <= x_s) then l_A supports all
//             of A and B with B strictly above it, so a_{i+1} stays a vertex: alpha > i;
//             otherwise l_B supports everything with A strictly above it: beta < k.
// Each step removes the candidate and one side of at least one range, so it ends after
// O(log) steps per range.  lo/hi bound the ranges known to contain alpha and beta.
// Returns false if the ranges run empty (possible only through rounding), leaving the outputs
// unspecified; the caller then finishes by walking.
template <class VS>
ISO_HD bool bridge_search(const VS& S, const NodeList& LA, const NodeList& LB, VRef loA, VRef hiA,
                          VRef loB, VRef hiB, const GPt& Sp, VRef& alpha, VRef& beta) {
  const VRef firstA = list_first(LA), lastA = list_last(LA);
  const VRef firstB = list_succ(LB, list_first(LB));  // first vertex of B without s
  const VRef lastB = list_last(LB);
  for (int it = 0; it < 4096; ++it) {
    if (!vref_le(loA, hiA) || !vref_le(loB, hiB)) return false;
    VRef i = list_mid(LA, loA, hiA);
    VRef k = list_mid(LB, loB, hiB);
    GPt a = load_v(S, LA, i);
    GPt b = load_v(S, LB, k);
    bool hasPA = !vref_eq(i, firstA), hasSA = !vref_eq(i, lastA);
    bool hasPB = !vref_eq(k, firstB), hasSB = !vref_eq(k, lastB);
    VRef pi{}, si{}, pk{}, sk{};
    GPt pa{}, sa{}, pb{}, sb{};
    bool Ab = false, Aa = false, Bb = false, Ba = false;
    if (hasPA) {
      pi = list_pred(LA, i);
      pa = load_v(S, LA, pi);
      Ab = !gleft(pa, a, b);
    }
    if (!Ab && hasSA) {
      si = list_succ(LA, i);
      sa = load_v(S, LA, si);
      Aa = gleft(a, sa, b);
    }
    if (hasSB) {
      sk = list_succ(LB, k);
      sb = load_v(S, LB, sk);
      Bb = !gleft(a, b, sb);
    }
    if (!Bb && hasPB) {
      pk = list_pred(LB, k);
      pb = load_v(S, LB, pk);
      Ba = gleft(a, pb, b);
    }
    bool Ac = !Ab && !Aa, Bc = !Bb && !Ba;
    if (Ac && Bc) {
      alpha = i;
      beta = k;
      return true;
    }
    if (Ab) {
      if (vref_eq(i, loA)) return false;
      hiA = pi;
    }
    if (Bb) {
      if (vref_eq(k, hiB)) return false;
      loB = sk;
    }
    if (Aa && Bc) loA = si;
    if (Ac && Ba) hiB = pk;
    if (Aa && Ba) {
      // Heights of s above l_A and above l_B, scaled by the edges' widths:
      //   h_A = turn(a_i, a_{i+1}, s) / dxA,  h_B = turn(b_{k-1}, b_k, s) / dxB.
      // l_B(x_s) >= l_A(x_s)  <=>  h_B <= h_A  <=>  turnB * dxA <= turnA * dxB (double-double).
      const DD dxA = gdx_dd(a, sa), dxB = gdx_dd(pb, b);
      const DD tA = gturn_dd(a, sa, Sp), tB = gturn_dd(pb, b, Sp);
      if (dd_sub(dd_mul(tA, dxB), dd_mul(tB, dxA)).hi >= 0.0) {
        loA = si;
      } else {
        hiB = pk;
      }
    }
  }
  return false;
}

// ------------------------------------------------------------------ reconstruction

// Per chunk, from the root list (Corollary 4.5): the chunk's surviving vertex range and the
// slopes of the edges into and out of it; a chunk with no segment lies under one edge.
struct EndInfo {
  int lo, hi;     // surviving vertex positions of the chunk's hull, or -1
  int klo, khi;   // their point indices within the chunk
  double sin;     // slope of the edge into vertex lo (or of the single covering edge)
  double sout;    // slope of the edge out of vertex hi
  int p0v;        // the chunk's point 0 is a vertex of the row's hull
  int pad[3];
};

template <class VS>
ISO_HD EndInfo chunk_ends(const VS& S, int64_t row, int j) {
  const int64_t rb = row * S.m;
  const int64_t g = rb + j;
  const Desc* root = S.desc + rb;
  const int nr = S.nseg[rb];
  // the root segment of the last chunk <= j: bracket it from a guess (exact when every chunk
  // keeps a segment), then bisect
  int lo = 0, hi = nr - 1;  // root[0].x == 0 <= j
  {
    int u0 = (int)(((int64_t)j * nr) / S.m);
    u0 = u0 < 0 ? 0 : (u0 > nr - 1 ? nr - 1 : u0);
    if (root[u0].x <= j) {
      lo = u0;
      int step = 1;
      while (lo + step <= hi && root[lo + step].x <= j) {
        lo += step;
        step <<= 1;
      }
      if (lo + step <= hi) hi = lo + step - 1;
    } else {
      hi = u0 - 1;  // the answer is below u0; probe downwards with doubling steps
      int probe = u0 - 1, step = 1;
      while (probe > 0 && root[probe].x > j) {
        hi = probe - 1;
        probe -= step;
        step <<= 1;
        if (probe < 0) probe = 0;
      }
      if (root[probe].x <= j) lo = probe;
    }
  }
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (root[mid].x <= j) lo = mid;
    else hi = mid - 1;
  }
  const int u = lo;
  const Desc du = root[u];
  EndInfo e;
  e.pad[0] = e.pad[1] = e.pad[2] = 0;
  if (du.x == j) {
    e.lo = du.y;
    e.hi = du.z;
    const double4 sj = S.start[g];
    const GPt plo = S.make_gpt(S.local(row, j, du.y, e.klo), sj);
    const GPt phi = S.make_gpt(S.local(row, j, du.z, e.khi), sj);
    e.sin = 0.0;
    e.sout = 0.0;
    if (u > 0) {
      const Desc dp = root[u - 1];
      e.sin = gslope(S.pt(row, dp.x, dp.z), plo);
    }
    if (u + 1 < nr) {
      const Desc dn = root[u + 1];
      e.sout = gslope(phi, S.pt(row, dn.x, dn.y));
    }
    int p0 = (du.y == 0) ? 1 : 0;
    if (!p0 && u > 0 && j > 0) {
      const Desc dp = root[u - 1];
      if (dp.x == j - 1 && dp.z == S.nverts[g - 1] - 1) p0 = 1;
    }
    e.p0v = p0;
  } else {
    // root[u + 1] exists: the row's last chunk always keeps a segment.
    e.lo = e.hi = -1;
    e.klo = e.khi = 0;
    const Desc dn = root[u + 1];
    const double s = gslope(S.pt(row, du.x, du.z), S.pt(row, dn.x, dn.y));
    e.sin = s;
    e.sout = s;
    e.p0v = (j > 0 && du.x == j - 1 && du.z == S.nverts[g - 1] - 1) ? 1 : 0;
  }
  return e;
}

}  // namespace iso
