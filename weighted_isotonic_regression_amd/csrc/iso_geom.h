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
//   Section 6 "Coordinates"  chunk-relative coordinates plus double-double chunk starts, so
//                that differences of nearby points keep their precision.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define ISO_HD __host__ __device__ __forceinline__

namespace iso {

constexpr int kWave = 64;                    // lanes of a wavefront
constexpr int kLanePts = 32;                 // elements per lane of a packed short-row tile
constexpr int kShortMax = 4 * kWave * kLanePts;  // rows of at most this many go to the short-row kernel
constexpr int kSub = 256;                    // points per lane of a long-row chunk
constexpr int kChunk = kWave * kSub;         // elements per chunk of a long row (one wavefront)
constexpr int kCk = 32;                      // spacing of a lane's running-sum checkpoints
constexpr int kLaneW = kSub / kCk;           // mask words (and checkpoints) per lane
constexpr int kSubW = kLaneW + 1;            // mask words of a lane's points 0..256
constexpr int kListCap = 256;                // chunks with at most this many hull vertices keep a list
constexpr int kMaskW = kChunk / 32 + 1;      // mask words of a chunk (points 0..16384)
constexpr int kZTiles = kChunk / 8;          // load tiles of a chunk (at least 8 elements each)
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

// Sign-exact comparison helper: sign of (a*b - c*d) for exactly representable factors whose
// products may exceed 2^53 (used by the separator test of the bridge search).
ISO_HD double diff_of_products(double a, double b, double c, double d) {
  double p1 = a * b;
  double e1 = fma(a, b, -p1);
  double p2 = c * d;
  double e2 = fma(c, d, -p2);
  return (p1 - p2) + (e1 - e2);
}

// ------------------------------------------------------------------ lane hull

// Monotone chain over the points 0..c of one lane (c <= 32), read through P(k, &x, &y).
// Returns the hull as a bit mask (bit k set iff point k is a vertex).  A point is popped when
// the turn (under, top, next) is <= 0, so collinear middle points are dropped.  Every iteration
// either pops or pushes, and exactly one point load is issued per iteration.
template <class PtFn>
ISO_HD uint64_t lane_chain(int c, PtFn P) {
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
    double t = cross2(tx - ux, ty - uy, kx - ux, ky - uy);
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
// [a0, s], node B spans [s, b1]; vertices are set bits of M, coordinates come from P.
// The bridge (alpha, beta) is found with alpha the leftmost contact in A (s included) and beta
// the rightmost contact in B \ {s}; the bits strictly between them are cleared.
template <class PtFn>
ISO_HD void tile_walk_merge(uint32_t* M, int a0, int s, int b1, PtFn P) {
  int al = s;
  int be = mask_succ(M, s);
  double ax, ay, bx, by;
  P(al, ax, ay);
  P(be, bx, by);
  // Each move removes a vertex of A or B, so the total number of moves is below b1 - a0.
  for (int pass = 0; pass <= b1 - a0; ++pass) {
    bool moved = false;
    while (al != a0) {
      int p = mask_pred(M, al);
      double px, py;
      P(p, px, py);
      if (cross2(ax - px, ay - py, bx - px, by - py) <= 0.0) {
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
      if (cross2(bx - ax, by - ay, qx - ax, qy - ay) <= 0.0) {
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

// A point in row coordinates: chunk-relative (x, y) plus the chunk's double-double start.
struct GPt {
  double x, y;
  double sxh, sxl, syh, syl;
};

// q - p with the coordinate hierarchy: the start difference first (exact for nearby chunks by
// Sterbenz's lemma), then the local difference.  For two points of one chunk the starts cancel
// to exactly zero and the result is the local difference.
ISO_HD void gdiff(const GPt& p, const GPt& q, double& dx, double& dy) {
  dx = ((q.sxh - p.sxh) + (q.sxl - p.sxl)) + (q.x - p.x);
  dy = ((q.syh - p.syh) + (q.syl - p.syl)) + (q.y - p.y);
}

ISO_HD double gturn(const GPt& a, const GPt& b, const GPt& c) {
  double dx1, dy1, dx2, dy2;
  gdiff(a, b, dx1, dy1);
  gdiff(a, c, dx2, dy2);
  return cross2(dx1, dy1, dx2, dy2);
}

ISO_HD double gslope(const GPt& a, const GPt& b) {
  double dx, dy;
  gdiff(a, b, dx, dy);
  return dy / dx;
}

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
//   list   the vertices' chunk-relative coordinates and chunk point indices, in order (hulls of
//          at most kListCap vertices whose coordinates the chunk pass had at hand);
//   dense  the vertex bit mask of the chunk's points 0..16384, the number of set bits before
//          each word, the lane starts and every lane's running sums at each 32nd point.  A
//          vertex's coordinates are recomputed from these and the inputs with the same fp64
//          operations in the same order as the chunk pass, so they are bitwise its values.
// Dense chunks are the ones whose points nearly all survive; storing them as lists would move
// about 18 bytes per element, while the dense form takes under one.
template <typename T, bool W, bool D>
struct VertexStore {
  Desc* desc;             // [G] descriptor slots
  int* nseg;              // [G] length of the list of the node starting at this slot
  const int* nverts;      // [G] vertex count of each chunk hull
  const uint8_t* dense;   // [G] 0 list form, 1 dense form, 2 dense form of an all-vertex chunk
  const double* lx;       // [G * kListCap] list form
  const double* ly;
  const uint16_t* lk;
  const uint32_t* mask;   // [G * kMaskW] dense form
  const uint16_t* mcnt;   // [G * kMaskW]
  const double* lsx;      // [G * kWave]  lane starts (weighted only)
  const double* lsy;      // [G * kWave]
  const double* ckx;      // [G * kWave * kLaneW] lane-relative running sums (weighted only)
  const double* cky;
  const double2* tot;     // [G] chunk end point (W, S)
  const double4* start;   // [G] chunk start {x hi, x lo, y hi, y lo}
  const double4* bnd;     // [G] dense form: coordinates of vertices 1 and V - 2
  const int2* bndk;       // [G] their point indices
  const T* y;
  const T* w;
  int64_t n;              // row length
  int m;                  // chunks per row

  ISO_HD bool is_list(int64_t g) const { return dense[g] == 0; }

  // Chunk-relative coordinates of point k (0..len) of dense chunk j of `row`.
  ISO_HD void dense_point(int64_t row, int j, int k, double& x, double& yy) const {
    const int64_t g = row * m + j;
    const int64_t rem = n - (int64_t)j * kChunk;
    const int len = rem < kChunk ? (int)rem : kChunk;
    if (k == len) {
      const double2 t = tot[g];
      x = t.x;
      yy = t.y;
      return;
    }
    const int l = k / kSub, q = k % kSub;
    const double sx = W ? lsx[g * kWave + l] : (double)(kSub * l);
    const double sy = lsy[g * kWave + l];
    if (q == 0) {
      x = sx;
      yy = sy;
      return;
    }
    const int jj = q / kCk;
    const int64_t cb = (g * kWave + l) * kLaneW + jj;
    double ax = W ? ckx[cb] : 0.0, ay = cky[cb];
    const int64_t e0 = row * n + (int64_t)j * kChunk + (int64_t)l * kSub;
    for (int e = kCk * jj; e < q; ++e) {
      double wd = W ? (double)w[e0 + e] : 1.0;
      double yd = yval<D>(y[e0 + e]);
      if (!isfinite(yd) || !isfinite(wd) || !(wd > 0.0)) {
        yd = 0.0;
        wd = 1.0;
      }
      if (W) ax += wd;
      ay += wd * yd;
    }
    x = W ? sx + ax : (double)k;
    yy = sy + ay;
  }

  // Lane start (sx, sy) and lane-relative running sums (ax, ay) at point k (0 <= k < len) of
  // dense chunk j: point k is (W ? sx + ax : k, sy + ay), with the operations of dense_point, so
  // adding elements k, k + 1, ... to (ax, ay) in order gives dense_point's values of the points
  // after k up to the next multiple of 32.
  ISO_HD void dense_state(int64_t row, int j, int k, double& sx, double& sy, double& ax, double& ay) const {
    const int64_t g = row * m + j;
    const int l = k / kSub, q = k % kSub;
    sx = W ? lsx[g * kWave + l] : (double)(kSub * l);
    sy = lsy[g * kWave + l];
    ax = 0.0;
    ay = 0.0;
    if (q == 0) return;
    const int jj = q / kCk;
    const int64_t cb = (g * kWave + l) * kLaneW + jj;
    if (W) ax = ckx[cb];
    ay = cky[cb];
    const int64_t e0 = row * n + (int64_t)j * kChunk + (int64_t)l * kSub;
    for (int e = kCk * jj; e < q; ++e) {
      double wd = W ? (double)w[e0 + e] : 1.0;
      double yd = yval<D>(y[e0 + e]);
      if (!isfinite(yd) || !isfinite(wd) || !(wd > 0.0)) {
        yd = 0.0;
        wd = 1.0;
      }
      if (W) ax += wd;
      ay += wd * yd;
    }
  }

  // Chunk-relative coordinates and point index of vertex p of chunk j of `row`.
  ISO_HD void local(int64_t row, int j, int p, double& x, double& yy, int& k) const {
    const int64_t g = row * m + j;
    if (dense[g] == 0) {
      const int64_t idx = g * kListCap + p;
      x = lx[idx];
      yy = ly[idx];
      k = lk[idx];
      return;
    }
    // the vertices the merges and ends touch most: the chunk's two ends and their neighbours
    const int V = nverts[g];
    if (p == 0) {
      x = 0.0;
      yy = 0.0;
      k = 0;
      return;
    }
    if (p == V - 1) {
      const int64_t rem = n - (int64_t)j * kChunk;
      k = rem < kChunk ? (int)rem : kChunk;
      const double2 t = tot[g];
      x = t.x;
      yy = t.y;
      return;
    }
    if (p == 1 || p == V - 2) {
      const double4 b = bnd[g];
      const int2 bk = bndk[g];
      if (p == 1) {
        x = b.x;
        yy = b.y;
        k = bk.x;
      } else {
        x = b.z;
        yy = b.w;
        k = bk.y;
      }
      return;
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
    dense_point(row, j, k, x, yy);
  }

  // pt() for a chunk known to be in list form (one round of independent loads).
  ISO_HD GPt pt_list(int64_t row, int j, int p) const {
    const int64_t g = row * m + j;
    const int64_t idx = g * kListCap + p;
    GPt r;
    r.x = lx[idx];
    r.y = ly[idx];
    const double4 s = start[g];
    r.sxh = s.x;
    r.sxl = s.y;
    r.syh = s.z;
    r.syl = s.w;
    return r;
  }

  // pt() of vertex p of the chunk of descriptor d, whose form and vertex count the descriptor
  // carries: list vertices and the dense form's cached ones need one round of loads.
  ISO_HD GPt pt_desc(int64_t row, const Desc& d, int p) const {
    const int form = desc_form(d), V = desc_nverts(d);
    if (form == 0) return pt_list(row, d.x, p);
    const int64_t g = row * m + d.x;
    if (p == 0 || p == V - 1 || p == 1 || p == V - 2) {
      GPt r;
      const double4 s = start[g];
      r.sxh = s.x;
      r.sxl = s.y;
      r.syh = s.z;
      r.syl = s.w;
      if (p == 0) {
        r.x = 0.0;
        r.y = 0.0;
      } else if (p == V - 1) {
        const double2 t = tot[g];
        r.x = t.x;
        r.y = t.y;
      } else {
        const double4 b = bnd[g];
        r.x = p == 1 ? b.x : b.z;
        r.y = p == 1 ? b.y : b.w;
      }
      return r;
    }
    return pt(row, d.x, p);
  }

  ISO_HD GPt pt(int64_t row, int j, int p) const {
    GPt r;
    int k;
    local(row, j, p, r.x, r.y, k);
    const double4 s = start[row * m + j];
    r.sxh = s.x;
    r.sxl = s.y;
    r.syh = s.z;
    r.syl = s.w;
    return r;
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
      Ab = gturn(pa, a, b) <= 0.0;
    }
    if (!Ab && hasSA) {
      si = list_succ(LA, i);
      sa = load_v(S, LA, si);
      Aa = gturn(a, sa, b) > 0.0;
    }
    if (hasSB) {
      sk = list_succ(LB, k);
      sb = load_v(S, LB, sk);
      Bb = gturn(a, b, sb) <= 0.0;
    }
    if (!Bb && hasPB) {
      pk = list_pred(LB, k);
      pb = load_v(S, LB, pk);
      Ba = gturn(a, pb, b) > 0.0;
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
      // l_B(x_s) >= l_A(x_s)  <=>  h_B <= h_A  <=>  turnB * dxA <= turnA * dxB.
      double dxA, dyA, dxB, dyB;
      gdiff(a, sa, dxA, dyA);
      gdiff(pb, b, dxB, dyB);
      double tA = gturn(a, sa, Sp);
      double tB = gturn(pb, b, Sp);
      if (diff_of_products(tA, dxB, tB, dxA) >= 0.0) {
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
    GPt plo = S.pt(row, j, du.y);
    GPt phi = S.pt(row, j, du.z);
    double tx, ty;
    S.local(row, j, du.y, tx, ty, e.klo);
    S.local(row, j, du.z, tx, ty, e.khi);
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
