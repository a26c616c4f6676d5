// iso_chunk.h -- the chunk pass of long rows on gfx950: one wavefront per chunk of 16384 elements,
// each lane running the monotone chain over its own 256 consecutive points.
//
// "Merge Hulls Without Copying Vertices: GPU Isotonic Regression":
//   Section 3.1  a lane builds the lower hull of its consecutive points by the monotone chain
//                (pop while the turn is not strictly left, so collinear middle points go).  The
//                page gives a lane 32 points; here a lane takes 256, so the 64 lanes of a wave
//                run 64 independent chains and the chunk needs only six merge rounds.
//   Section 3.2  the lane hulls of the chunk merge pairwise in rounds; the first lane of each
//                right half walks to the bridge (Lemma 4.2).  A lane's surviving vertices are
//                always one contiguous range of its stack, so a round only cuts ranges.  From
//                groups of eight lanes on, a group whose stacks are shallow first runs both walks
//                on a register window of the vertices next to the shared point, a ballot per
//                move, and walks on serially only if a walk leaves the window.
//   Section 3.3  the chunk's hull is emitted for the merge levels, as a vertex list when it is
//                small and as a bit mask with coordinate checkpoints when it is dense.
//   Section 6    "Coordinates": a lane works in coordinates relative to its first point; the
//                chunk-relative coordinates are its start (a double-double wave scan of the lane
//                totals) plus those.  Running sums are pairs (hi, lo): hi is the fp64 running sum
//                the chain works with, lo the exact sum of its rounding errors.
//   Section 6    "Predicates": a turn of the chain is evaluated on the hi parts and used when it
//                exceeds an a-priori bound built from the magnitudes of its own differences and
//                products and of the lo parts; a chunk with a turn inside its bound is processed
//                again by an exact pass, which decides such turns in double-double arithmetic
//                from the three points' pairs, recomputed from their checkpoints.
//
// Per lane state: the top three stack entries in registers, the last kRingS entries in an LDS
// ring indexed by depth, the stack as a bit mask in LDS, and the running sums every 32 points (the
// checkpoints).  An entry that has left the ring is found again from the mask and recomputed
// from its checkpoint and the inputs; on the measured workloads this is rare (the stacks of noisy
// rows stay shallow and dense rows never pop).
//
// In the first pass a lane does not pop at the element that causes the pops: its candidate points
// wait in a short LDS queue, and after each element the wave runs chain steps (one push or pop
// per lane) only while some queue is full, so that lanes with few pops are not held at every
// element by the lane with the most.  A point joins the queue only if it can be a vertex at all:
// y_{q-1} < y_q, and it passes two exact tests against its second neighbours (Lemma 4.1 lets any
// stage drop its own non-vertices).  The exact pass keeps the plain element-by-element chain.
//
// Dense rows: a clean strictly increasing tile pushed on top of its two predecessors has every
// element as its own block so far, so the lane writes z = y for it and marks the tile.  The fit
// pass keeps those values where the final hull confirms single-element blocks (Corollary 4.5)
// and writes the rest.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "iso_geom.h"
#include "iso_kernels.h"

namespace iso {

// Per-chunk outputs of the chunk pass.
struct ChunkOut {
  // Each array of lo parts follows its array of hi parts in the same allocation (G chunks apart),
  // so that only the hi pointers are passed.
  double2* tot;       // [2G] chunk end point (W, S), chunk-relative: hi parts, then lo parts
  int* nverts;        // [G] vertex count of the chunk hull
  uint32_t* cflags;   // [G] input flags of the chunk
  Desc* desc;         // [G] leaf segment list
  int* nseg;          // [G]
  uint16_t* lk;       // [G * kListCap] list form: chunk point index
  double* lx;         // [2G * kListCap] chunk-relative pairs: hi parts, then lo parts
  double* ly;
  uint32_t* mask;     // [G * kMaskW] dense form: vertex bits of chunk points 0..16384
  uint16_t* mcnt;     // [G * kMaskW] set bits before each word
  double* lsx;        // [2G * kWave] lane starts (chunk-relative pairs)
  double* lsy;
  double* ckx;        // [2G * kLaneW * kWave] lane-relative running sums at points 32 j (pairs),
                      //     [j * kWave + lane] within a chunk, so a wave's stores are contiguous
  double* cky;
  uint32_t* ztile;    // [G * kWave] per lane: bit t set where the lane chain wrote z = y for its
                      //     elements 8 t .. 8 t + 7
  uint8_t* dform;     // [G] 0 list form, 1 dense form, 2 dense form with every point a vertex
                      //     and z = y written for the whole chunk, 3 not yet processed
  double4* bnd;       // [2G] dense form: coordinates of hull vertices 1 and V - 2 (hi, then lo)
  int2* bndk;         // [G] their point indices
  int64_t G;          // chunks of the call

  __device__ double2* totl() const { return tot + G; }
  __device__ double* lxl() const { return lx + G * kListCap; }
  __device__ double* lyl() const { return ly + G * kListCap; }
  __device__ double* lsxl() const { return lsx + G * kWave; }
  __device__ double* lsyl() const { return lsy + G * kWave; }
  __device__ double* ckxl() const { return ckx + G * (kWave * kLaneW); }
  __device__ double* ckyl() const { return cky + G * (kWave * kLaneW); }
  __device__ double4* bndl() const { return bnd + G; }
};

__device__ __forceinline__ double turn_pts(double2 p, double2 q, double2 r) {
  return cross2(q.x - p.x, q.y - p.y, r.x - p.x, r.y - p.y);
}

// Lanes strictly below lane x (x in 0..64).
__device__ __forceinline__ uint64_t lanes_below(int x) {
  return x >= 64 ? ~0ull : ((1ull << x) - 1ull);
}

// Nearest integer in the input's own precision (an integer test needs no conversion).
__device__ __forceinline__ float rint_t(float v) { return rintf(v); }
__device__ __forceinline__ double rint_t(double v) { return rint(v); }

// c ? a : b on values (never on references, so both sides stay in registers).
__device__ __forceinline__ double sel(bool c, double a, double b) { return c ? a : b; }
__device__ __forceinline__ int sel(bool c, int a, int b) { return c ? a : b; }

// One input element as the chain uses it: a non-finite value or a weight <= 0 is replaced by
// (y, w) = (0, 1), and its kind is or-ed into f.
template <bool W>
__device__ __forceinline__ void classify(double& yd, double& wd, uint32_t& f) {
  uint32_t fk = 0u;
  if (!isfinite(yd) || !isfinite(wd)) fk = ISO_ROW_NONFINITE_BIT;
  else if (!(wd > 0.0)) fk = ISO_ROW_BAD_WEIGHT_BIT;
  if (fk) {
    f |= fk;
    yd = 0.0;
    wd = 1.0;
  }
}

// Stack entries a lane keeps in LDS: depths 0 and 1 have slots of their own, deeper entries cycle
// through kRingS - 2 slots.  Every slot carries a tag (point index and depth), so a read knows
// whether the slot still holds the entry of the depth it asks for; an entry that has been
// overwritten is found again from the stack mask and recomputed from its checkpoint and the
// inputs.
constexpr int kRingS = 12;

template <bool W>
struct RingCoord {
  using type = double2;  // lane-relative (x, y)
};
template <>
struct RingCoord<false> {
  using type = double;  // y only: x is the point index
};

// The first pass's candidate queue: a lane's points waiting for the chain, kQ slots per lane.  The
// elements stream through kQStep at a time; before the next kQStep points can arrive, every lane
// must hold at most kQ - kQStep, so the wave runs chain steps (one push or one pop per lane) only
// while some lane is above that.  A lane with few pops thus runs ahead of the others instead of
// waiting at every element for the lane with the most.
constexpr int kQ = 4;
constexpr int kQStep = 1;

// Merge rounds from this one on (groups of 2^r lanes) first walk in a register window.
constexpr int kWinRound = 3;
constexpr int kWinDepth = 32;

// LDS of one wavefront.  The queue is used only during the chains and the lane results only
// after them, so they share their space.
template <bool W>
struct ChunkLds {
  typename RingCoord<W>::type ring[kRingS][kWave];
  uint16_t rtag[kRingS][kWave];
  uint32_t smask[kSubW][kWave];  // stack bit mask over the lane's points 0..256
  union {
    struct {
      int depth[kWave];              // final stack depth
      int lo[kWave], hi[kWave];      // surviving depth range of the lane's stack
      double2 start[kWave + 1];      // lane starts, chunk-relative (hi); [l + 1] is lane l's end point
      double2 startl[kWave + 1];     // (lo)
      uint32_t wa[kWave], wb[kWave]; // merge-round windows: (lane << 16 | depth) of the vertices next to s
    };
    struct {
      typename RingCoord<W>::type qp[kQ][kWave];  // queued points, lane-relative (y only without w)
      uint8_t qi[kQ][kWave];                      // their point indices less one
    };
  };
};


// Ring slot of stack depth i.
__device__ __forceinline__ int ring_slot(int i) { return i < 2 ? i : 2 + (i - 2) % (kRingS - 2); }

// Slot of depth i + 1 from the slot s of depth i, and of depth i - 1 from the slot s of depth i.
__device__ __forceinline__ int ring_next(int s) { return s == kRingS - 1 ? 2 : s + 1; }
__device__ __forceinline__ int ring_prev(int s, int i) { return (s == 2 && i > 2) ? kRingS - 1 : s - 1; }

// A slot's tag: point index q (9 bits) and depth i mod 128.  Slots are reused only by depths that
// differ by multiples of the ring's cycle (kRingS - 2 = 10), so two depths of one slot below 640
// never share a residue mod 128: the tag tells the depth exactly.
__device__ __forceinline__ uint32_t ring_tag(int q, int i) { return (uint32_t)q | ((uint32_t)(i & 127) << 9); }
__device__ __forceinline__ int tag_q(uint32_t tg) { return (int)(tg & 0x1ffu); }
__device__ __forceinline__ bool tag_is(uint32_t tg, int i) { return (tg >> 9) == (uint32_t)(i & 127); }

template <bool W>
__device__ __forceinline__ void ring_put(ChunkLds<W>& L, int s, int lane, double x, double y,
                                         uint32_t tag) {
  if constexpr (W) L.ring[s][lane] = double2{x, y};
  else L.ring[s][lane] = y;
  L.rtag[s][lane] = (uint16_t)tag;
}

// Reads slot s of lane l: point index q, lane-relative coordinates, and whether the slot holds
// the entry of depth i (tag and coordinates are read together, whatever the answer).
template <bool W>
__device__ __forceinline__ bool ring_get(const ChunkLds<W>& L, int s, int l, int i, int& q,
                                         double& x, double& y) {
  const uint32_t tg = L.rtag[s][l];
  const typename RingCoord<W>::type P = L.ring[s][l];
  q = tag_q(tg);
  if constexpr (W) {
    x = P.x;
    y = P.y;
  } else {
    x = (double)q;
    y = P;
  }
  return tag_is(tg, i);
}

// Lane-relative coordinates of lane l's point q, from the checkpoint below q and the inputs (the
// same operations in the same order as the chain).  ck = the chunk's checkpoints.
template <typename T, bool W, bool D>
__device__ double2 lane_point(const double* ckx, const double* cky, int l, int q, int c,
                              const T* yl, const T* wl) {
  q = min(max(q, 0), c);
  const int j = min(q / kCk, kLaneW - 1);
  double2 P{W ? ckx[j * kWave + l] : 0.0, cky[j * kWave + l]};
  uint32_t f = 0u;
  for (int e = kCk * j; e < q; ++e) {
    double yd = yval<D>(yl[e]), wd = W ? (double)wl[e] : 1.0;
    classify<W>(yd, wd, f);
    if (W) P.x += wd;
    P.y += wd * yd;
  }
  if (!W) P.x = (double)q;
  return P;
}

// Lane-relative pairs of lane l's point q, from the checkpoint pairs below q and the inputs (the
// chain's operations in its order, so its hi parts are lane_point's).
template <typename T, bool W, bool D>
__device__ __forceinline__ PD lane_point_dd(const double* ckx, const double* cky, const double* ckxl,
                                            const double* ckyl, int l, int q, int c, const T* yl, const T* wl) {
  constexpr bool EX = ExactProd<T, W>::value;
  q = min(max(q, 0), c);
  const int j = min(q / kCk, kLaneW - 1);
  DD ax{0.0, 0.0}, ay{cky[j * kWave + l], ckyl[j * kWave + l]};
  if (W) ax = DD{ckx[j * kWave + l], ckxl[j * kWave + l]};
  uint32_t f = 0u;
  for (int e = kCk * j; e < q; ++e) {
    double yd = yval<D>(yl[e]), wd = W ? (double)wl[e] : 1.0;
    classify<W>(yd, wd, f);
    if (W) acc(ax.hi, ax.lo, wd);
    acc_prod<EX>(ay.hi, ay.lo, wd, yd);
  }
  if (!W) ax = DD{(double)q, 0.0};
  return PD{ax, ay};
}

// Turn (U, T, K) of lane l's stack entries U = point ui and T = point ti (recomputed from their
// checkpoints) and K, the lane's running sums (kx + kxl, ky + kyl), in double-double arithmetic.
// Out of line: the chain reaches it only when its fast turn is inside the error bound.
template <typename T, bool W, bool D>
__device__ __noinline__ double chain_turn_dd(const double* ckx, const double* cky, const double* ckxl,
                                             const double* ckyl, int l, int ui, int ti, int c, const T* yl,
                                             const T* wl, double kx, double kxl, double ky, double kyl) {
  const PD Up = lane_point_dd<T, W, D>(ckx, cky, ckxl, ckyl, l, ui, c, yl, wl);
  const PD Tp = lane_point_dd<T, W, D>(ckx, cky, ckxl, ckyl, l, ti, c, yl, wl);
  return turn_dd(Up, Tp, PD{DD{kx, kxl}, DD{ky, kyl}}).hi;
}

// Stack mask word ww of lane l; the word the chain is filling (cw) is still in a register.
template <bool W>
__device__ __forceinline__ uint32_t mask_word(const ChunkLds<W>& L, int l, int ww, int wi,
                                              uint32_t curw) {
  return ww == wi ? curw : L.smask[ww][l];
}

// Point index of the stack entry at depth i of lane l (after the chain: the whole mask is in
// LDS): the ring's tag, else the i-th set bit (from 0) of the stack mask.  The stack holds more
// than i entries, so the bit exists; the clamp keeps later reads inside the lane.
template <bool W>
__device__ int lane_index(const ChunkLds<W>& L, int l, int i, int c, bool& in_ring) {
  in_ring = false;
  if (i == 0) return 0;
  const int s = ring_slot(i);
  const uint32_t tg = L.rtag[s][l];
  if (tag_is(tg, i)) {
    in_ring = true;
    return tag_q(tg);
  }
  int rem = i;
  int wd = 0;
  for (; wd < kSubW - 1; ++wd) {
    const int pc = __popc(L.smask[wd][l]);
    if (rem < pc) break;
    rem -= pc;
  }
  uint32_t word = L.smask[wd][l];
  for (int r = 0; r < rem && word; ++r) word &= word - 1u;
  const int q = word ? kCk * wd + __builtin_ctz(word) : 0;
  return min(q, c);
}

// Point index q and lane-relative coordinates of the stack entry at depth i of lane l.
template <typename T, bool W, bool D>
__device__ double2 lane_entry(const ChunkLds<W>& L, const double* ckx, const double* cky, int l,
                              int i, int c, const T* yl, const T* wl, int& q) {
  bool in_ring;
  q = lane_index<W>(L, l, i, c, in_ring);
  if (i == 0) return double2{0.0, 0.0};
  if (in_ring) {
    double x, yy;
    (void)ring_get<W>(L, ring_slot(i), l, i, q, x, yy);
    return double2{x, yy};
  }
  return lane_point<T, W, D>(ckx, cky, l, q, c, yl, wl);
}

// Chunk-relative coordinates and point index q (0..256, within the lane) of the stack entry at
// depth i of lane l.
template <typename T, bool W, bool D>
__device__ __forceinline__ double2 chunk_entry(const ChunkLds<W>& L, const double* ckx,
                                               const double* cky, int l, int i, int len,
                                               const T* yc, const T* wc, int& q) {
  const int c = min(max(len - kSub * l, 0), kSub);
  if (i == 0) {
    q = 0;
    return L.start[l];
  }
  if (i == L.depth[l] - 1) {
    q = c;
    return L.start[l + 1];
  }
  const double2 P = lane_entry<T, W, D>(L, ckx, cky, l, i, c, yc + kSub * l,
                                     W ? wc + kSub * l : nullptr, q);
  const double2 S = L.start[l];
  return double2{W ? S.x + P.x : (double)(kSub * l + q), S.y + P.y};
}

template <typename T, bool W, bool D>
__device__ __forceinline__ double2 chunk_entry(const ChunkLds<W>& L, const double* ckx,
                                               const double* cky, int l, int i, int len,
                                               const T* yc, const T* wc) {
  int q;
  return chunk_entry<T, W, D>(L, ckx, cky, l, i, len, yc, wc, q);
}

// Chunk-relative pairs of the stack entry at depth i of lane l: the lane's start, its end point
// (the next lane's start) or the start plus the entry's lane-relative pairs.
template <typename T, bool W, bool D>
__device__ PD chunk_entry_dd(const ChunkLds<W>& L, const double* ckx, const double* cky, const double* ckxl,
                             const double* ckyl, int l, int i, int len, const T* yc, const T* wc, int& q) {
  const int c = min(max(len - kSub * l, 0), kSub);
  if (i == 0 || i == L.depth[l] - 1) {
    const int ls = i == 0 ? l : l + 1;
    q = i == 0 ? 0 : c;
    return PD{DD{L.start[ls].x, L.startl[ls].x}, DD{L.start[ls].y, L.startl[ls].y}};
  }
  bool in_ring;
  q = lane_index<W>(L, l, i, c, in_ring);
  const PD a = lane_point_dd<T, W, D>(ckx, cky, ckxl, ckyl, l, q, c, yc + kSub * l, W ? wc + kSub * l : nullptr);
  return VertexStore<T, W, D>::join(DD{L.start[l].x, L.startl[l].x}, DD{L.start[l].y, L.startl[l].y}, a.x, a.y,
                                    kSub * l + q);
}

// Turn of three stack entries (lane, depth) of the chunk's lanes from their chunk-relative pairs.
template <typename T, bool W, bool D>
__device__ __forceinline__ double entries_turn_dd(const ChunkLds<W>& L, const double* ckx, const double* cky,
                                                  const double* ckxl, const double* ckyl, const int (&ls)[3],
                                                  const int (&is)[3], int len, const T* yc, const T* wc) {
  PD Q[3];
#pragma unroll 1
  for (int k = 0; k < 3; ++k) {
    int q;
    Q[k] = chunk_entry_dd<T, W, D>(L, ckx, cky, ckxl, ckyl, ls[k], is[k], len, yc, wc, q);
  }
  return turn_dd(Q[0], Q[1], Q[2]).hi;
}

// Chunks whose elements are all clean and strictly increasing.  Every turn of such a chunk's
// diagram compares two consecutive y values, so every point P_0 .. P_len is a strict vertex of the
// chunk hull: the hull is the whole diagram and every element is its own block.  A workgroup of
// kIncWaves wavefronts streams the chunk's len elements with coalesced nontemporal 16-byte loads
// and stores (wavefront q takes the q-th of kIncWaves equal parts), checks the pattern, writes
// z = y and stores the dense form directly: vertex bits of points 0..len set, lane starts,
// checkpoints (here double-double block sums accumulated in a fixed order; every later coordinate
// of the chunk is computed from these stored pairs), and the cache of vertices 1 and V - 2
// computed exactly as the stored-form readers recompute points.  It keeps no z tile marks: form 2 itself tells the
// fit that z = y holds for every element.  It returns false, having written only z, when an
// element breaks the pattern; the lane chains then process the chunk and rewrite everything.
// Requires len >= 2 * kCk and 16-byte aligned y, w, z.  bs: LDS for the 512 block sums (pairs of x
// and y); bad: an int of LDS.
constexpr int kIncWaves = 4;

struct BlockSums {
  double x[kChunk / kCk], xl[kChunk / kCk], y[kChunk / kCk], yl[kChunk / kCk];
};

template <typename T, bool W, bool D>
__device__ bool increasing_chunk(const T* __restrict__ yc, const T* __restrict__ wc,
                                 T* __restrict__ zc, int len, int64_t g, int j,
                                 const ChunkOut& out, BlockSums& bs, int* bad) {
  constexpr bool EX = ExactProd<T, W>::value;
  constexpr int VN = Vec16<T>::N;
  constexpr int U = 4;                   // vectors per lane per step
  constexpr int SE = kWave * VN * U;     // elements per step of one wavefront
  constexpr int BL = kCk / VN;           // lanes per 32-element block
  constexpr int QE = kChunk / kIncWaves; // elements per wavefront
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x >> 6;
  if (threadIdx.x == 0) *bad = 0;
  {
    // probe: the first kIncWaves 16-byte vectors of each of the wavefront's lane segments (noisy
    // rows fail here, and the lines read are the ones the lane chains read first)
    constexpr int SPW = kWave / kIncWaves;  // lane segments per wavefront
    bool ok = true;
    const int e = kSub * (SPW * wv + (lane % SPW)) + VN * (lane / SPW);
    if (e + VN <= len) {
      T pv[VN];
      load16(yc + e, pv);
      const double before = (lane / SPW) ? yval<D>(yc[e - 1]) : -INFINITY;
      double prev = before;
#pragma unroll
      for (int k = 0; k < VN; ++k) {
        const double yd = yval<D>(pv[k]);
        ok = ok && isfinite(yd) && prev < yd;
        prev = yd;
      }
    }
    if (__syncthreads_or(!ok)) return false;
  }
  const int q0 = QE * wv, q1 = min(QE * (wv + 1), len);
  double carry = q0 > 0 && q0 < len ? yval<D>(yc[q0 - 1]) : -INFINITY;
  for (int s0 = q0; s0 < q1; s0 += SE) {
    T yv[U * VN], wv_[U * VN];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = s0 + (u * kWave + lane) * VN;
      if (e + VN <= q1) {
        load16_nt(yc + e, &yv[u * VN]);
        if (W) load16_nt(wc + e, &wv_[u * VN]);
      } else {
#pragma unroll
        for (int k = 0; k < VN; ++k) {
          yv[u * VN + k] = e + k < q1 ? yc[e + k] : (T)0;
          if (W) wv_[u * VN + k] = e + k < q1 ? wc[e + k] : (T)0;
        }
      }
    }
    bool ok = true;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = s0 + (u * kWave + lane) * VN;
      const double last = yval<D>(yv[u * VN + VN - 1]);
      double prev = __shfl_up(last, 1, kWave);
      if (lane == 0) prev = carry;
      DD sw{0.0, 0.0}, sy{0.0, 0.0};
#pragma unroll
      for (int k = 0; k < VN; ++k) {
        if (e + k < q1) {
          const double yd = yval<D>(yv[u * VN + k]);
          const double wd = W ? (double)wv_[u * VN + k] : 1.0;
          ok = ok && isfinite(yd) && isfinite(wd) && wd > 0.0 && prev < yd;
          prev = yd;
          if (W) acc(sw.hi, sw.lo, wd);
          acc_prod<EX>(sy.hi, sy.lo, wd, yd);
        }
      }
      carry = __shfl(last, kWave - 1, kWave);
      // block sums: a DPP butterfly over the block's BL lanes (every lane of a block ends with
      // the same pair)
      if (W) sw = group_pair_sum<BL>(sw);
      sy = group_pair_sum<BL>(sy);
      if ((lane & (BL - 1)) == 0 && e < q1) {
        if (W) {
          bs.x[e / kCk] = sw.hi;
          bs.xl[e / kCk] = sw.lo;
        }
        bs.y[e / kCk] = sy.hi;
        bs.yl[e / kCk] = sy.lo;
      }
      if (e + VN <= q1) {
        store16_nt(zc + e, &yv[u * VN]);
      } else {
#pragma unroll
        for (int k = 0; k < VN; ++k)
          if (e + k < q1) zc[e + k] = yv[u * VN + k];
      }
    }
    if (!__all(ok)) {
      if (lane == 0) *bad = 1;
      break;
    }
    if (*(volatile int*)bad) break;  // another wavefront failed (seen late at worst)
  }
  if (__syncthreads_or(*bad)) return false;
  if (wv != 0) return true;
  // wavefront 0 stores the form.  Lane l: checkpoints of its points (exclusive sums of its eight
  // blocks; a block past len sums to zero) and its total; jv = the block of point len - 1 in the
  // lane that holds it
  const int kv = len - 1, lv = kv / kSub, jv = (kv % kSub) / kCk;
  DD cx{0.0, 0.0}, cy{0.0, 0.0}, cvx{0.0, 0.0}, cvy{0.0, 0.0};
  const int64_t cb = g * (int64_t)(kWave * kLaneW) + lane;
#pragma unroll
  for (int jj = 0; jj < kLaneW; ++jj) {
    if (W) {
      out.ckx[cb + jj * kWave] = cx.hi;
      out.ckxl()[cb + jj * kWave] = cx.lo;
    }
    out.cky[cb + jj * kWave] = cy.hi;
    out.ckyl()[cb + jj * kWave] = cy.lo;
    if (jj == jv) {
      cvx = cx;
      cvy = cy;
    }
    const int bi = kLaneW * lane + jj;
    if (kCk * bi < len) {
      if (W) cx = dd_add(cx, DD{bs.x[bi], bs.xl[bi]});
      cy = dd_add(cy, DD{bs.y[bi], bs.yl[bi]});
    }
  }
  // lane starts: double-double wave scan of the lane totals
  DD ix = cx, iy = cy;
#pragma unroll
  for (int dd = 1; dd < kWave; dd <<= 1) {
    const DD vx{__shfl_up(ix.hi, dd, kWave), __shfl_up(ix.lo, dd, kWave)};
    const DD vy{__shfl_up(iy.hi, dd, kWave), __shfl_up(iy.lo, dd, kWave)};
    if (lane >= dd) {
      ix = dd_add(vx, ix);
      iy = dd_add(vy, iy);
    }
  }
  DD sx{__shfl_up(ix.hi, 1, kWave), __shfl_up(ix.lo, 1, kWave)};
  DD sy{__shfl_up(iy.hi, 1, kWave), __shfl_up(iy.lo, 1, kWave)};
  if (lane == 0) {
    sx = DD{0.0, 0.0};
    sy = DD{0.0, 0.0};
  }
  if (!W) sx = DD{(double)(kSub * lane), 0.0};
  if (W) {
    out.lsx[g * kWave + lane] = sx.hi;
    out.lsxl()[g * kWave + lane] = sx.lo;
  }
  out.lsy[g * kWave + lane] = sy.hi;
  out.lsyl()[g * kWave + lane] = sy.lo;
  // vertex bits of points 0..len, set bits before each word
  const int64_t mb = g * (int64_t)kMaskW;
#pragma unroll
  for (int wd = 0; wd < kLaneW; ++wd) {
    const int w0 = kCk * (kLaneW * lane + wd);  // the word's first point
    uint32_t bits = 0u;
    if (w0 + 31 <= len) bits = 0xffffffffu;
    else if (w0 <= len) bits = (2u << (len - w0)) - 1u;
    out.mask[mb + kLaneW * lane + wd] = bits;
    out.mcnt[mb + kLaneW * lane + wd] = (uint16_t)min(w0, len + 1);
  }
  if (lane == 0) {
    // vertex 1 = point 1: lane 0's start and checkpoint 0 (zero) plus element 0
    const double w0 = W ? (double)wc[0] : 1.0;
    DD ax{0.0, 0.0}, ay{0.0, 0.0};
    if (W) acc(ax.hi, ax.lo, w0);
    acc_prod<EX>(ay.hi, ay.lo, w0, yval<D>(yc[0]));
    const PD P = VertexStore<T, W, D>::join(sx, sy, ax, ay, 1);
    out.bnd[g].x = P.x.hi;
    out.bnd[g].y = P.y.hi;
    out.bndl()[g].x = P.x.lo;
    out.bndl()[g].y = P.y.lo;
    out.bndk[g].x = 1;
    out.nverts[g] = len + 1;
    out.desc[g] = make_int4(j, 0, len, desc_w(2, len + 1));
    out.nseg[g] = 1;
    out.cflags[g] = 0u;
    out.dform[g] = 2;
  }
  if (lane == kWave - 1) {
    out.mask[mb + kMaskW - 1] = len == kChunk ? 1u : 0u;  // point 16384
    out.mcnt[mb + kMaskW - 1] = (uint16_t)min(kChunk, len + 1);
    out.tot[g] = make_double2(W ? ix.hi : (double)len, iy.hi);
    out.totl()[g] = make_double2(W ? ix.lo : 0.0, iy.lo);
  }
  if (lane == lv) {
    // vertex V - 2 = point len - 1: this lane's checkpoint below it plus its elements from the
    // checkpoint on, in order (all loads issued before the first add)
    DD ax = cvx, ay = cvy;
    const int e0v = kSub * lv + kCk * jv;
    T ye[kCk - 1], we[kCk - 1];
#pragma unroll
    for (int k = 0; k < kCk - 1; ++k) {
      ye[k] = e0v + k < kv ? yc[e0v + k] : (T)0;
      we[k] = (W && e0v + k < kv) ? wc[e0v + k] : (T)1;
    }
#pragma unroll
    for (int k = 0; k < kCk - 1; ++k) {
      if (e0v + k < kv) {
        const double wd = W ? (double)we[k] : 1.0;
        if (W) acc(ax.hi, ax.lo, wd);
        acc_prod<EX>(ay.hi, ay.lo, wd, yval<D>(ye[k]));
      }
    }
    const PD P = (kv % kSub == 0) ? PD{sx, sy} : VertexStore<T, W, D>::join(sx, sy, ax, ay, kv);
    out.bnd[g].z = P.x.hi;
    out.bnd[g].w = P.y.hi;
    out.bndl()[g].z = P.x.lo;
    out.bndl()[g].w = P.y.lo;
    out.bndk[g].y = kv;
  }
  return true;
}

// Runs before k_chunk: one workgroup per chunk tries increasing_chunk on chunks of at least 64
// elements whose inputs are 16-byte aligned, and marks the chunk's form byte 2 when it succeeds,
// 3 otherwise (k_chunk then processes the chunk and writes its form).
template <typename T, bool W, bool D>
__global__ __launch_bounds__(kIncWaves * kWave) void k_increasing(const T* __restrict__ y,
                                                                  const T* __restrict__ w,
                                                                  T* __restrict__ z, int64_t n,
                                                                  int m, ChunkOut out) {
  __shared__ BlockSums bs;
  __shared__ int bad;
  const int64_t g = blockIdx.x;
  const int64_t row = g / m;
  const int j = (int)(g - row * m);
  const int64_t off = row * n + (int64_t)j * kChunk;
  const int64_t rem = n - (int64_t)j * kChunk;
  const int len = rem < kChunk ? (int)rem : kChunk;
  const bool vec = (((uintptr_t)(y + off)) % 16 == 0) && (!W || ((uintptr_t)(w + off)) % 16 == 0) &&
                   (((uintptr_t)(z + off)) % 16 == 0);
  bool done = false;
  if (len >= 2 * kCk && vec)
    done = increasing_chunk<T, W, D>(y + off, W ? w + off : nullptr, z + off, len, g, j, out, bs, &bad);
  if (!done && threadIdx.x == 0) out.dform[g] = 3;
}

template <typename T, bool W, bool D, bool EXACT>
__global__ __launch_bounds__(64, W ? 2 : 3) void k_chunk(const T* __restrict__ y,
                                                        const T* __restrict__ w,
                                                        T* __restrict__ z, int64_t n, int m,
                                                        ChunkOut out) {
  __shared__ ChunkLds<W> L;
  constexpr bool EX = ExactProd<T, W>::value;
  constexpr int TN = Tile<T, W>::N;  // elements per load tile
  constexpr int VN = Vec16<T>::N;
  const int lane = threadIdx.x;
  const int64_t g = blockIdx.x;
  const int64_t row = g / m;
  const int j = (int)(g - row * m);
  const int64_t off = row * n + (int64_t)j * kChunk;
  const int64_t rem = n - (int64_t)j * kChunk;
  const int len = rem < kChunk ? (int)rem : kChunk;
  const int e0 = kSub * lane;
  const int c = min(max(len - e0, 0), kSub);         // elements of this lane
  const int nl = (len + kSub - 1) / kSub;            // lanes holding elements
  const bool vec = (((uintptr_t)(y + off)) % 16 == 0) && (!W || ((uintptr_t)(w + off)) % 16 == 0) &&
                   (((uintptr_t)(z + off)) % 16 == 0);
  const T* yc = y + off;  // the chunk's inputs
  const T* wc = W ? w + off : nullptr;
  const T* yl = yc + e0;  // the lane's
  const T* wl = W ? wc + e0 : nullptr;
  T* zl = z + off + e0;
  double* ckx = out.ckx + g * (int64_t)(kWave * kLaneW);  // the chunk's checkpoints
  double* cky = out.cky + g * (int64_t)(kWave * kLaneW);
  double* ckxl = out.ckxl() + g * (int64_t)(kWave * kLaneW);
  double* ckyl = out.ckyl() + g * (int64_t)(kWave * kLaneW);
  // done by k_increasing (form 2), or by the first pass (forms 0 and 1)
  if (EXACT ? out.dform[g] != 3 : out.dform[g] == 2) return;
  if (EXACT && lane == 0) atomicAdd(&g_branch_counts[2], 1ull);

  // ---- a1-a3: stream the lane's elements through the chain.  Point P_q (0 < q < c) lies between
  // the elements q - 1 and q, whose slopes are y_{q-1} and y_q; unless y_{q-1} < y_q it is not a
  // strict vertex of any hull containing its neighbours, so it is never pushed.
  for (int wd = 0; wd < kSubW; ++wd) L.smask[wd][lane] = 0u;
  for (int sl = 0; sl < kRingS; ++sl) L.rtag[sl][lane] = 0xffffu;
  uint32_t f = 0u;
  // The top three stack entries T (depth d - 1), U (d - 2) and V (d - 3) are held in registers
  // with their point indices ti, ui, vi and ring slots ts, us, vs.
  int d = 0;
  double tx = 0.0, ty = 0.0, ux = 0.0, uy = 0.0, vx = 0.0, vy = 0.0;
  double lx = 0.0, ly = 0.0;     // running sums (hi)
  double lxl = 0.0, lyl = 0.0;   // their lo parts
  double aabs = 0.0;             // sum of |w y| so far: bounds every |y| of the lane's points
  double lomx = 0.0, lomy = 0.0; // largest |lo| of the running sums so far
  double yprev = 0.0;
  bool undec = false;      // a turn of the first pass fell inside its error bound
  double frac = 0.0;       // 0 while every coordinate so far is an integer
  uint32_t ztb = 0u;       // z-tile marks of the lane's elements
  const int ntiles = (c + TN - 1) / TN;
  if constexpr (EXACT) {
    int ti = 0, ui = 0, vi = 0, ts = 0, us = 0, vs = 0;
    int wi = 0;
    uint32_t curw = 0u;
    if (c > 0) {  // point 0 at depth 0
      ring_put<W>(L, 0, lane, 0.0, 0.0, ring_tag(0, 0));
      d = 1;
      curw = 1u;
    }
    int pops = 0;
    // V is refilled from the ring after each pop (depth d - 3); its tag is checked only when the
    // next pop is about to make it U, so the LDS read overlaps the next turn.  An overwritten entry
    // is recomputed: the highest stack bit below ui, from its checkpoint and the inputs; that
    // recomputation waits for its own loads before it leaves, so no load of it is still pending
    // where the loop continues.
    uint32_t vtag = 0u;
    bool vchk = false;
    auto check_v = [&]() {
      if (!vchk) return;
      vi = tag_q(vtag);
      if (!W) vx = (double)vi;
      if (d >= 3 && !tag_is(vtag, d - 3)) {
        int ww = ui >> 5;
        uint32_t mw = mask_word<W>(L, lane, ww, wi, curw) & ((1u << (ui & 31)) - 1u);
        while (mw == 0u) {
          --ww;
          mw = mask_word<W>(L, lane, ww, wi, curw);
        }
        vi = kCk * ww + 31 - __builtin_clz(mw);
        const double2 P = lane_point<T, W, D>(ckx, cky, lane, vi, c, yl, wl);
        vx = P.x;
        vy = P.y;
        __builtin_amdgcn_s_waitcnt(0);
      }
      vchk = false;
    };
    // The exact pass (the chunks the first pass left).  The turn (U, T, K) is first taken on the
    // hi parts.  Every point so far has 0 <= x <= Ax (the current x), |y| <= Ay = sum |w y|, and
    // lo parts of at most LX and LY in magnitude (the largest seen), so each difference of hi parts
    // is within u |d| + 2 LX (or 2 LY) of the difference of the pairs and the fast turn is within
    // 14 u Ax Ay + 4 Ax LY + 8 Ay LX (to first order) of the turn of the pairs; Ecur = 16 u Ax Ay +
    // 8 (Ax LY + Ay LX), set before each push.  While every point pushed so far has integer
    // coordinates below 2^25 (frac = 0, Ax and Ay below 2^25), the fast turn is exact.  Otherwise
    // a turn inside the bound is decided in double-double arithmetic from U and T recomputed from
    // their checkpoints and K's running pairs.
    double Ecur = 0.0;
    auto turn_utk = [&](const double kx, const double ky, const int q) {
      double t = cross2(tx - ux, ty - uy, kx - ux, ky - uy);
      const bool ilane = frac == 0.0 && (W ? lx : (double)q) < 0x1p25 && aabs < 0x1p25;
      if (d >= 2 && !ilane && !(fabs(t) > Ecur))
        t = chain_turn_dd<T, W, D>(ckx, cky, ckxl, ckyl, lane, ui, ti, c, yl, wl, kx, W ? lxl : 0.0, ky, lyl);
      return t;
    };
    // pushes point q with lane-relative coordinates (kx, ky), first popping what it makes
    // non-convex (pop while the turn (U, T, K) is not strictly left).  A popped entry's stack bit
    // is cleared in LDS (the word being filled is rewritten from curw later) and in curw.
    auto push = [&](const double kx, const double ky, const int q) {
      {
        const double ax = W ? lx : (double)q;
        Ecur = fma(ax * 0x1p-49, aabs, 8.0 * fma(ax, lomy, aabs * lomx));
      }
      frac = fmax(frac, fabs(ky - floor(ky)) + (W ? fabs(kx - floor(kx)) : 0.0));
      bool more = (d >= 2) & !(turn_utk(kx, ky, q) > 0.0);
      if (more) {
        while (more) {
          check_v();
          {
            const uint32_t nbit = ~(1u << (ti & 31));
            atomicAnd(&L.smask[ti >> 5][lane], nbit);
            if ((ti >> 5) == wi) curw &= nbit;
          }
          ++pops;
          tx = ux;
          ty = uy;
          ti = ui;
          ts = us;
          ux = vx;
          uy = vy;
          ui = vi;
          us = vs;
          --d;
          vs = max(ring_prev(us, d - 2), 0);
          const uint32_t tg = L.rtag[vs][lane];
          if constexpr (W) {
            const double2 P = L.ring[vs][lane];
            vx = P.x;
            vy = P.y;
          } else {
            vy = L.ring[vs][lane];
          }
          vtag = tg;  // (the point index and the check wait until V is used)
          vchk = true;
          more = (d >= 2) & !(turn_utk(kx, ky, q) > 0.0);
        }
      }
      const int ks = ring_next(ts);
      ring_put<W>(L, ks, lane, kx, ky, ring_tag(q, d));
      curw |= 1u << (q & 31);
      vx = ux;
      vy = uy;
      vi = ui;
      vs = us;
      ux = tx;
      uy = ty;
      ui = ti;
      us = ts;
      tx = kx;
      ty = ky;
      ti = q;
      ts = ks;
      vchk = false;
      ++d;
    };
    // the next tile's inputs are loaded while the current one is processed
    T ny[TN], nw[TN];
    auto load_tile = [&](int eb) {
      if (vec && eb + TN <= c) {
  #pragma unroll
        for (int k = 0; k < TN / VN; ++k) {
          load16(yl + eb + k * VN, &ny[k * VN]);
          if (W) load16(wl + eb + k * VN, &nw[k * VN]);
        }
      } else {
  #pragma unroll
        for (int k = 0; k < TN; ++k) {
          ny[k] = (eb + k < c) ? yl[eb + k] : (T)0;
          if (W) nw[k] = (eb + k < c) ? wl[eb + k] : (T)1;
        }
      }
    };
    if (ntiles > 0) load_tile(0);
    for (int t = 0; t < ntiles; ++t) {
      const int eb = t * TN;  // lane-relative index of the tile's first element
      if ((eb & (kCk - 1)) == 0) {
        if (W) {
          ckx[(eb / kCk) * kWave + lane] = lx;
          ckxl[(eb / kCk) * kWave + lane] = lxl;
        }
        cky[(eb / kCk) * kWave + lane] = ly;
        ckyl[(eb / kCk) * kWave + lane] = lyl;
      }
      if ((eb >> 5) != wi) {  // the tile's points 32 w .. are in mask word w (same for every lane)
        L.smask[wi][lane] = curw;
        wi = eb >> 5;
        curw = 0u;
      }
      T yv[TN], wv[TN];
  #pragma unroll
      for (int k = 0; k < TN; ++k) {
        yv[k] = ny[k];
        wv[k] = W ? nw[k] : (T)1;
      }
      if (t + 1 < ntiles) load_tile(eb + TN);
      const int kn = min(TN, c - eb);
      // Tile checks.  A non-finite value or a weight <= 0 is replaced by (y, w) = (0, 1) and its
      // kind recorded.  When the tile's elements are clean and strictly increasing in y after the
      // previous element, every turn among its points and the two before them is strictly convex
      // in exact arithmetic (the slopes of the one-element edges are the y values), so once the
      // stack's top two entries are the points just before the tile's (the first of them was
      // pushed on top of its own predecessor, so its turn is convex too), all of the tile's points
      // are pushed without tests.
      bool clean = kn == TN, incr = true;
      {
        double yp = yprev;
  #pragma unroll
        for (int k = 0; k < TN; ++k) {
          const double yd = yval<D>(yv[k]);
          const double wd = W ? (double)wv[k] : 1.0;
          clean = clean && isfinite(yd) && isfinite(wd) && wd > 0.0;
          incr = incr && (yp < yd || (eb == 0 && k == 0));
          yp = yd;
        }
      }
      if (!__all(clean)) {
  #pragma unroll
        for (int k = 0; k < TN; ++k) {
          if (k < kn) {
            double yd = (double)yv[k], wd = W ? (double)wv[k] : 1.0;
            classify<W>(yd, wd, f);
            yv[k] = (T)yd;
            if (W) wv[k] = (T)wd;
          }
        }
      }
      const int pops0 = pops;
      bool skipped = false;
      // one element through the chain: its left point q (a candidate when y_{q-1} < y_q), then
      // the running sums
      auto element = [&](int k) {
        const double yd = yval<D>(yv[k]);
        const double wd = W ? (double)wv[k] : 1.0;
        const int q = eb + k;
        if (q > 0) {
          if (yprev < yd) push(W ? lx : (double)q, ly, q);
          else skipped = true;
        }
        if (W) acc(lx, lxl, wd);
        const double p = wd * yd;
        if constexpr (EX) acc(ly, lyl, p);
        else acc_pe(ly, lyl, p, fma(wd, yd, -p));
        aabs += fabs(p);
        if (W) lomx = fmax(lomx, fabs(lxl));
        lomy = fmax(lomy, fabs(lyl));
        yprev = yd;
      };
      // pushes the tile's points eb + k, k >= kp, without tests, and consumes its elements k >= kc
      // (point eb + k is pushed before element k is added to the running sums)
      auto bulk_push = [&](const int kp, const int kc) {
        int s = ts;
  #pragma unroll
        for (int k = 0; k < TN; ++k) {
          if (k >= kp) {
            const double kx = W ? lx : (double)(eb + k), ky = ly;
            frac = fmax(frac, fabs(ky - floor(ky)) + (W ? fabs(kx - floor(kx)) : 0.0));
            s = ring_next(s);
            if (k >= TN - (kRingS - 2) || d < 2) ring_put<W>(L, s, lane, kx, ky, ring_tag(eb + k, d));
            vx = ux;
            vy = uy;
            vi = ui;
            vs = us;
            ux = tx;
            uy = ty;
            ui = ti;
            us = ts;
            tx = kx;
            ty = ky;
            ti = eb + k;
            ts = s;
            ++d;
          }
          if (k >= kc) {
            const double wd = W ? (double)wv[k] : 1.0;
            const double yd = yval<D>(yv[k]);
            if (W) acc(lx, lxl, wd);
            const double p = wd * yd;
            if constexpr (EX) acc(ly, lyl, p);
            else acc_pe(ly, lyl, p, fma(wd, yd, -p));
            aabs += fabs(p);
            if (W) lomx = fmax(lomx, fabs(lxl));
            lomy = fmax(lomy, fabs(lyl));
          }
        }
        yprev = yval<D>(yv[TN - 1]);
        const int b0 = (eb & 31) + kp, b1 = (eb & 31) + TN - 1;  // bits of points eb+kp .. eb+TN-1
        curw |= (b1 >= 31 ? 0xffffffffu : ((2u << b1) - 1u)) & ~((1u << b0) - 1u);
      };
      // bulk from the tile's first point, or else after element 0 went through the chain (at
      // eb == 0, d == 1 means point 0 alone on the stack)
      bool bulk = __all(clean && incr && (eb == 0 ? d == 1 : (ti == eb - 1 && ui == eb - 2)));
      int kp = eb == 0 ? 1 : 0, kc = 0;
      if (!bulk) {
        if (kn > 0) element(0);
        bulk = __all(clean && incr && ti == eb && (eb == 0 ? d == 1 : ui == eb - 1));
        kp = 1;
        kc = 1;
      }
      if (bulk) {
        bulk_push(kp, kc);
      } else {
  #pragma unroll
        for (int k = 1; k < TN; ++k)
          if (k < kn) element(k);
      }
      // speculative fit of a tile that pushed every point and popped none: every element is its
      // own block so far
      uint8_t zt = 0;
      if (pops == pops0 && !skipped && kn == TN && vec) {
  #pragma unroll
        for (int k = 0; k < TN / VN; ++k) store16(zl + eb + k * VN, &yv[k * VN]);
        zt = 1;
      }
#pragma unroll
      for (int h = 0; h < TN / kZT; ++h) ztb |= (uint32_t)zt << (eb / kZT + h);
    }
    if (c > 0) {
      // the lane's end point (and its checkpoint when it starts a checkpoint block, so that every
      // point of the lane has one)
      if ((c & (kCk - 1)) == 0 && c < kSub) {
        if (W) {
          ckx[(c / kCk) * kWave + lane] = lx;
          ckxl[(c / kCk) * kWave + lane] = lxl;
        }
        cky[(c / kCk) * kWave + lane] = ly;
        ckyl[(c / kCk) * kWave + lane] = lyl;
      }
      if ((c >> 5) != wi) {
        L.smask[wi][lane] = curw;
        wi = c >> 5;
        curw = 0u;
      }
      push(W ? lx : (double)c, ly, c);
      L.smask[wi][lane] = curw;
    }
  } else {
    // The first pass.  Each lane queues its candidate points in LDS as the elements stream
    // through, and the wave runs chain steps on the queues whenever a lane's queue is about to
    // overflow.  A turn is decided by the sign of its fp64 value on the hi parts when that value
    // exceeds its error bound, built from the magnitudes of the differences and products it is
    // made of (below); a chunk with a turn inside its bound is left to the exact pass, unless
    // every input so far is an integer and the sums stay below 2^25, which makes every turn exact.
    int ti = 0, ui = 0, vi = 0, ts = 0, us = 0, vs = 0;
    if (c > 0) {  // point 0 at depth 0
      ring_put<W>(L, 0, lane, 0.0, 0.0, ring_tag(0, 0));
      L.smask[0][lane] = 1u;
      d = 1;
    }
    int qh = 0, qt = 0;  // queue head and tail counters (slot = counter mod kQ)
    // K = the queue's head and N = the entry after it, read one step ahead
    double kx = 0.0, ky = 0.0, nx = 0.0, ny_ = 0.0;
    int kq = 0, nq = 0;
    bool intin = true;   // every input so far an integer
    // Error bound of the turn (U, T, K) computed as p1 - p2, p1 = dx1 dy2, p2 = dy1 dx2, with
    // (dx1, dy1) = T - U and (dx2, dy2) = K - T on the hi parts.  A hi part is within LX (LY) of its
    // pair (the largest |lo| so far), so each difference is within u|d| + 2 LX (or LY) of the
    // difference of the pairs; with the rounding of the two products and the subtraction, the
    // turn of the pairs is within 4u' (|p1| + |p2|) + 2 LX (|dy1| + |dy2|) + 2 LY (|dx1| + |dx2|)
    // + 8 LX LY of t, to first order; each term is taken 1 % larger for the neglected ones.
    double cLX = 0.0, cLY = 0.0, E0 = 0x1p-1000;
    bool dexact = false;  // every sum exact so far, but not the integer case below 2^25
    // After a pop, V's ring entry is read into (rvx, rvy, rtg) and taken into V only when the next
    // pop needs it (vpend), so the read overlaps a whole step.  An entry whose tag shows it was
    // overwritten is recomputed: the highest stack bit below ui, from its checkpoint and the
    // inputs (waiting for its own loads before it leaves).
    double rvx = 0.0, rvy = 0.0;
    uint32_t rtg = 0u;
    bool vpend = false;
    struct QE {
      double x, y;
      int q;
    };
    auto read_q = [&](const int h) __attribute__((always_inline)) {
      const int s = h & (kQ - 1);
      QE e;
      if constexpr (W) {
        const double2 P = L.qp[s][lane];
        e.x = P.x;
        e.y = P.y;
      } else {
        e.y = L.qp[s][lane];
      }
      e.q = (int)L.qi[s][lane] + 1;
      if (!W) e.x = (double)e.q;
      return e;
    };
    // one push or pop of the queue's head K, for every lane that has one
    auto step = [&]() __attribute__((always_inline)) {
      const bool act = qt != qh;
      const double dx1 = tx - ux, dy1 = ty - uy, dx2 = kx - tx, dy2 = ky - ty;
      const double p1 = dx1 * dy2, p2 = dy1 * dx2;
      const double t = p1 - p2;
      const double E = fma(4.04 * kU, fabs(p1) + fabs(p2),
                           fma(cLY, fabs(dx1) + fabs(dx2), fma(cLX, fabs(dy1) + fabs(dy2), E0)));
      // (bitwise operators throughout, so that the compiler keeps the step free of branches)
      const bool tst = act & (d >= 2);
      // While no running sum of the lane has rounded (every lo part so far is zero: LX = LY = 0)
      // the hi parts are the coordinates, and a turn inside its bound is decided here, in
      // double-double arithmetic on them, as the exact pass would (ties and collinear runs of
      // values that sum exactly, e.g. fp32 values of one binade in an fp64 row without weights,
      // which the soft rank's problems are).  Integer inputs below 2^25 need none of it: there
      // the fast turn is exact.  Only unweighted fp64 rows carry this code.
      bool und = false;
      double td = t;
      if constexpr (!W && sizeof(T) == 8) {  // (the soft rank's problems are of this kind)
        und = dexact & tst & !(fabs(t) > E);
        if (__any(und)) {
          if (und) {
            td = turn_dd(PD{DD{ux, 0.0}, DD{uy, 0.0}}, PD{DD{tx, 0.0}, DD{ty, 0.0}},
                         PD{DD{kx, 0.0}, DD{ky, 0.0}}).hi;
          }
        }
      }
      undec = undec | (tst & !und & !(fabs(t) > E));
      const bool push = act & ((d < 2) | (td > 0.0));
      const bool pop = act & !push;
      // the stack mask: a push sets K's bit, a pop clears T's (an idle lane xors zero)
      {
        const int mi = push ? kq : ti;
        atomicXor(&L.smask[mi >> 5][lane], act ? 1u << (mi & 31) : 0u);
      }
      // A pop makes V the new U: V is the entry read after the previous pop when that read is
      // pending (vpend), and an entry whose tag shows it was overwritten is recomputed first.
      const bool stale = pop & vpend & (d >= 3) & !tag_is(rtg, d - 3);
      if (__any(stale)) {
        if (stale) {
          int ww = ui >> 5;
          uint32_t mw = L.smask[ww][lane] & ((1u << (ui & 31)) - 1u);
          while (mw == 0u) {
            --ww;
            mw = L.smask[ww][lane];
          }
          const int q = kCk * ww + 31 - __builtin_clz(mw);
          const double2 P = lane_point<T, W, D>(ckx, cky, lane, q, c, yl, wl);
          rvx = P.x;
          rvy = P.y;
          rtg = ring_tag(q, d - 3);
          __builtin_amdgcn_s_waitcnt(0);
        }
      }
      if (push) {
        const int ks = ring_next(ts);
        ring_put<W>(L, ks, lane, kx, ky, ring_tag(kq, d));
        vx = ux;
        vy = uy;
        vi = ui;
        vs = us;
        ux = tx;
        uy = ty;
        ui = ti;
        us = ts;
        tx = kx;
        ty = ky;
        ti = kq;
        ts = ks;
        ++d;
        ++qh;
        vpend = false;
        kx = nx;
        ky = ny_;
        kq = nq;
      } else if (pop) {
        if (vpend) {
          vi = tag_q(rtg);
          vx = W ? rvx : (double)vi;
          vy = rvy;
        }
        tx = ux;
        ty = uy;
        ti = ui;
        ts = us;
        ux = vx;
        uy = vy;
        ui = vi;
        us = vs;
        --d;
        vs = max(ring_prev(us, d - 2), 0);
        vpend = true;
      }
      // the reads for the next steps: the entry after the head, and V's ring slot
      {
        const QE e = read_q(qh + 1);
        nx = e.x;
        ny_ = e.y;
        nq = e.q;
      }
      rtg = L.rtag[vs][lane];
      if constexpr (W) {
        const double2 P = L.ring[vs][lane];
        rvx = P.x;
        rvy = P.y;
      } else {
        rvy = L.ring[vs][lane];
      }
    };
    // chain steps until no lane holds more than `keep` queued points
    auto drain = [&](const int keep) __attribute__((always_inline)) {
      if (!__any(qt - qh > keep)) return;
      cLX = 2.02 * lomx;
      cLY = 2.02 * lomy;
      E0 = 8.08 * lomx * lomy + 0x1p-1000;
      dexact = lomx == 0.0 && lomy == 0.0 && !(intin && (W ? lx : 0.0) < 0x1p25 && aabs < 0x1p25);
      {
        const QE e = read_q(qh), e2 = read_q(qh + 1);
        kx = e.x;
        ky = e.y;
        kq = e.q;
        nx = e2.x;
        ny_ = e2.y;
        nq = e2.q;
      }
      do {
        step();
      } while (__any(qt - qh > keep));
    };
    // element k of the tile: its left point joins the queue when it is a candidate, then the
    // element joins the running sums
    T yv[TN], wv[TN];
    T ny[TN], nw[TN];  // the next tile's inputs (loaded while the current one is processed)
    int eb = 0, kn = 0;  // the tile's first element and its element count
    double ypp = 0.0, wpp = 1.0, wprev = 1.0;  // elements q - 2 and q - 1 (y_{q-1} is yprev)
    auto produce = [&](const int k) __attribute__((always_inline)) {
      const double yd = yval<D>(yv[k]);
      const double wd = W ? (double)wv[k] : 1.0;
      const int q = eb + k;
      // Point P_q with y_{q-1} < y_q is also not a vertex when it is not a strict vertex of
      // (P_{q-2}, P_q, P_{q+1}) or of (P_{q-1}, P_q, P_{q+2}), i.e. when the weighted mean of
      // elements q - 2 and q - 1 is at least y_q, or that of elements q and q + 1 at most y_{q-1}.
      // In terms of the inputs, with dq = y_q - y_{q-1} > 0: w_{q-2} (y_{q-2} - y_q) >= w_{q-1} dq,
      // or w_{q+1} (y_{q-1} - y_{q+1}) >= w_q dq.  Each side is a difference and a product, so
      // its computed value is within a factor (1 +- u)^2 of the exact one, and a side that exceeds
      // the other one taken 2^-50 larger (plus 2^-960 against underflow) exceeds it exactly; such
      // a point is left out of the queue (any hull that holds it and those neighbours has it
      // above a chord), which does not change the lane's hull.
      bool cand = (q > 0) & (yprev < yd);
      {
        const bool hasn = k + 1 < TN ? (k + 1 < kn) : (eb + TN < c);
        const double yn = yval<D>(k + 1 < TN ? yv[k + 1 < TN ? k + 1 : 0] : ny[0]);
        const double wn = W ? (double)(k + 1 < TN ? wv[k + 1 < TN ? k + 1 : 0] : nw[0]) : 1.0;
        const double dq = yd - yprev;
        const double tl = fma(W ? wprev * dq : dq, 0x1.0000000000004p0, 0x1p-960);
        const double tr = fma(W ? wd * dq : dq, 0x1.0000000000004p0, 0x1p-960);
        const double al = W ? wpp * (ypp - yd) : ypp - yd;
        const double ar = W ? wn * (yprev - yn) : yprev - yn;
        // (for fp32 inputs the sides are finite: w dq stays below 2^256)
        const bool xl = (q >= 2) & (al >= tl) & (sizeof(T) == 4 || tl < INFINITY);
        const bool xr = hasn & (ar >= tr) & (sizeof(T) == 4 || tr < INFINITY);
        cand = cand & !xl & !xr;
      }
      ypp = yprev;
      wpp = wprev;
      wprev = wd;
      // every lane writes the slot after its queue's tail, which is free (at most kQ - 1 points
      // wait when an element arrives); only a candidate moves the tail over it
      {
        const int s = qt & (kQ - 1);
        if constexpr (W) L.qp[s][lane] = double2{lx, ly};
        else L.qp[s][lane] = ly;
        L.qi[s][lane] = (uint8_t)(q - 1);
        qt += cand ? 1 : 0;
      }
      if (W) acc(lx, lxl, wd);
      const double p = wd * yd;
      if constexpr (EX) acc(ly, lyl, p);
      else acc_pe(ly, lyl, p, fma(wd, yd, -p));
      aabs += fabs(p);
      if (W) lomx = fmax(lomx, fabs(lxl));
      lomy = fmax(lomy, fabs(lyl));
      intin = intin & (yv[k] == rint_t(yv[k])) & (!W || wv[k] == rint_t(wv[k]));
      yprev = yd;
    };
    // pushes the tile's points eb + k, k >= kp, without tests (a clean strictly increasing tile
    // on top of its two predecessors, every queue empty), and consumes its elements k >= kc
    auto bulk_push = [&](const int kp, const int kc) __attribute__((always_inline)) {
      int s = ts;
#pragma unroll
      for (int k = 0; k < TN; ++k) {
        if (k >= kp) {
          const double px = W ? lx : (double)(eb + k), py = ly;
          s = ring_next(s);
          if (k >= TN - (kRingS - 2) || d < 2) ring_put<W>(L, s, lane, px, py, ring_tag(eb + k, d));
          vx = ux;
          vy = uy;
          vi = ui;
          vs = us;
          ux = tx;
          uy = ty;
          ui = ti;
          us = ts;
          tx = px;
          ty = py;
          ti = eb + k;
          ts = s;
          ++d;
        }
        if (k >= kc) {
          const double wd = W ? (double)wv[k] : 1.0;
          const double yd = yval<D>(yv[k]);
          if (W) acc(lx, lxl, wd);
          const double p = wd * yd;
          if constexpr (EX) acc(ly, lyl, p);
          else acc_pe(ly, lyl, p, fma(wd, yd, -p));
          aabs += fabs(p);
          if (W) lomx = fmax(lomx, fabs(lxl));
          lomy = fmax(lomy, fabs(lyl));
          intin = intin && yv[k] == rint_t(yv[k]) && (!W || wv[k] == rint_t(wv[k]));
        }
      }
      vpend = false;
      yprev = yval<D>(yv[TN - 1]);
      ypp = yval<D>(yv[TN - 2]);
      wprev = W ? (double)wv[TN - 1] : 1.0;
      wpp = W ? (double)wv[TN - 2] : 1.0;
      const int b0 = (eb & 31) + kp, b1 = (eb & 31) + TN - 1;  // bits of points eb+kp .. eb+TN-1
      atomicOr(&L.smask[eb >> 5][lane],
               (b1 >= 31 ? 0xffffffffu : ((2u << b1) - 1u)) & ~((1u << b0) - 1u));
    };
    auto load_tile = [&](int e) __attribute__((always_inline)) {
      if (vec && e + TN <= c) {
#pragma unroll
        for (int k = 0; k < TN / VN; ++k) {
          load16(yl + e + k * VN, &ny[k * VN]);
          if (W) load16(wl + e + k * VN, &nw[k * VN]);
        }
      } else {
#pragma unroll
        for (int k = 0; k < TN; ++k) {
          ny[k] = (e + k < c) ? yl[e + k] : (T)0;
          if (W) nw[k] = (e + k < c) ? wl[e + k] : (T)1;
        }
      }
    };
    if (ntiles > 0) load_tile(0);
    for (int t = 0; t < ntiles; ++t) {
      eb = t * TN;
      if ((eb & (kCk - 1)) == 0) {
        if (W) {
          ckx[(eb / kCk) * kWave + lane] = lx;
          ckxl[(eb / kCk) * kWave + lane] = lxl;
        }
        cky[(eb / kCk) * kWave + lane] = ly;
        ckyl[(eb / kCk) * kWave + lane] = lyl;
      }
#pragma unroll
      for (int k = 0; k < TN; ++k) {
        yv[k] = ny[k];
        wv[k] = W ? nw[k] : (T)1;
      }
      if (t + 1 < ntiles) load_tile(eb + TN);
      kn = min(TN, c - eb);
      // tile checks, as in the exact pass
      bool clean = kn == TN, incr = true;
      {
        double yp = yprev;
#pragma unroll
        for (int k = 0; k < TN; ++k) {
          const double yd = yval<D>(yv[k]);
          const double wd = W ? (double)wv[k] : 1.0;
          clean = clean && isfinite(yd) && isfinite(wd) && wd > 0.0;
          incr = incr && (yp < yd || (eb == 0 && k == 0));
          yp = yd;
        }
      }
      if (!__all(clean)) {
#pragma unroll
        for (int k = 0; k < TN; ++k) {
          if (k < kn) {
            double yd = (double)yv[k], wd = W ? (double)wv[k] : 1.0;
            classify<W>(yd, wd, f);
            yv[k] = (T)yd;
            if (W) wv[k] = (T)wd;
          }
        }
      }
      // a clean strictly increasing tile goes on the stack without tests once the queues are
      // empty and the top two entries are the points just before the tile (at eb == 0, point 0
      // alone); failing that, after its first point went through the chain
      bool bulk = false;
      int kc = 0;
      if (__all(clean && incr)) {
        drain(0);
        bulk = __all(eb == 0 ? d == 1 : (ti == eb - 1 && ui == eb - 2));
        if (!bulk) {
          produce(0);
          drain(0);
          kc = 1;
          bulk = __all(ti == eb && (eb == 0 ? d == 1 : ui == eb - 1));
        }
      }
      uint8_t zt = 0;
      if (bulk) {
        bulk_push(eb == 0 ? 1 : kc, kc);
        // every element of the tile is its own block so far
        if (kn == TN && vec) {
#pragma unroll
          for (int k = 0; k < TN / VN; ++k) store16(zl + eb + k * VN, &yv[k * VN]);
          zt = 1;
        }
      } else {
#pragma unroll
        for (int k = 0; k < TN; ++k) {
          if (k >= kc && k < kn) produce(k);
          if ((k & (kQStep - 1)) == kQStep - 1) drain(kQ - kQStep);
        }
      }
#pragma unroll
      for (int h = 0; h < TN / kZT; ++h) ztb |= (uint32_t)zt << (eb / kZT + h);
    }
    if (c > 0) {
      // the lane's end point (and its checkpoint when it starts a checkpoint block, so that every
      // point of the lane has one) joins the queue, and the queues are emptied
      if ((c & (kCk - 1)) == 0 && c < kSub) {
        if (W) {
          ckx[(c / kCk) * kWave + lane] = lx;
          ckxl[(c / kCk) * kWave + lane] = lxl;
        }
        cky[(c / kCk) * kWave + lane] = ly;
        ckyl[(c / kCk) * kWave + lane] = lyl;
      }
      const int s = qt & (kQ - 1);
      if constexpr (W) L.qp[s][lane] = double2{lx, ly};
      else L.qp[s][lane] = ly;
      L.qi[s][lane] = (uint8_t)(c - 1);
      ++qt;
    }
    drain(0);
    frac = intin ? 0.0 : 1.0;
  }
  out.ztile[g * (int64_t)kWave + lane] = ztb;

  // ---- lane starts: double-double wave scan of the lane totals (chunk-relative coordinates).
  DD ix = two_sum(lx, lxl), iy = two_sum(ly, lyl);
#pragma unroll
  for (int dd = 1; dd < kWave; dd <<= 1) {
    const DD vx{__shfl_up(ix.hi, dd, kWave), __shfl_up(ix.lo, dd, kWave)};
    const DD vy{__shfl_up(iy.hi, dd, kWave), __shfl_up(iy.lo, dd, kWave)};
    if (lane >= dd) {
      ix = dd_add(vx, ix);
      iy = dd_add(vy, iy);
    }
  }
  DD sx{__shfl_up(ix.hi, 1, kWave), __shfl_up(ix.lo, 1, kWave)};
  DD sy{__shfl_up(iy.hi, 1, kWave), __shfl_up(iy.lo, 1, kWave)};
  if (lane == 0) {
    sx = DD{0.0, 0.0};
    sy = DD{0.0, 0.0};
  }
  if (!W) {
    sx = DD{(double)e0, 0.0};
    ix = DD{(double)(e0 + c), 0.0};
  }
  L.start[lane] = double2{sx.hi, sy.hi};
  L.startl[lane] = double2{sx.lo, sy.lo};
  if (lane == nl - 1) {
    L.start[lane + 1] = double2{ix.hi, iy.hi};
    L.startl[lane + 1] = double2{ix.lo, iy.lo};
  }
  // bound of the in-chunk walks' fast turns: chunk-relative x in [0, Xc], |y| <= Yc
  double yc_abs = aabs;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) yc_abs += __shfl_xor(yc_abs, o, kWave);
  L.depth[lane] = d;
  int lo = 1, hi = d - 1;  // depth 0 is the previous lane's end point (lane 0: the chunk start)
  L.lo[lane] = lo;
  L.hi[lane] = hi;
  __syncthreads();

  // ---- a4: merge rounds.  Node A = lanes [g0, sB), node B = lanes [sB, g0 + size); their
  // shared point s is lane sB - 1's end point.  A's vertices: (g0, 0), then each lane's range;
  // B's: each lane's range, ending at lane lb's end point.
  //
  // A strict left turn of three stack entries: the fast turn of the chunk-relative hi parts when
  // it exceeds its error bound, else the turn of the pairs.  Each hi coordinate is within
  // ex = 259 u Xc (ey = 259 u Yc) of its pair (the start's lo, the lane sum's lo, the rounding of
  // the sum), so with (dx1, dy1) = P2 - P1, (dx2, dy2) = P3 - P2 the turn dx1 dy2 - dy1 dx2 of
  // the pairs is within 4u'(|p1| + |p2|) + 2 ex (|dy1| + |dy2|) + 2 ey (|dx1| + |dx2|) + 8 ex ey
  // of the computed one, each term taken 1 % larger.
  const double ex2 = (W ? L.start[nl].x : (double)len) * (2.02 * 259.0 * kU);
  const double ey2 = yc_abs * (2.02 * 259.0 * kU);
  const double E00 = 2.0 * ex2 * ey2 + 0x1p-1000;
  auto wleft = [&](int l1, int i1, double2 P1, int l2, int i2, double2 P2, int l3, int i3, double2 P3) {
    const double dx1 = P2.x - P1.x, dy1 = P2.y - P1.y, dx2 = P3.x - P2.x, dy2 = P3.y - P2.y;
    const double p1 = dx1 * dy2, p2 = dy1 * dx2;
    const double t = p1 - p2;
    const double Ew = fma(4.04 * kU, fabs(p1) + fabs(p2),
                          fma(ex2, fabs(dy1) + fabs(dy2), fma(ey2, fabs(dx1) + fabs(dx2), E00)));
    if (fabs(t) > Ew) return t > 0.0;
    const int ls[3] = {l1, l2, l3}, is[3] = {i1, i2, i3};
    return entries_turn_dd<T, W, D>(L, ckx, cky, ckxl, ckyl, ls, is, len, yc, wc) > 0.0;
  };
#pragma unroll 1
  for (int r = 1; r <= 6; ++r) {
    const int gsz = 1 << r, half = gsz >> 1;
    const int g0 = lane & ~(gsz - 1);
    const int sB = g0 + half;
    const bool merge = sB < nl;
    const uint64_t nzr = __ballot(lo <= hi);  // lanes with a non-empty range
    const int lb = min(g0 + gsz, nl) - 1;       // B's last lane
    int al = 0, ai = 0, bl = 0, bi = 0;
    bool settled = false, from_win = false;
    if (r >= kWinRound) {
      // Only groups whose lanes' stacks are shallow (depth <= kWinDepth, as on noisy rows) walk
      // in a window: their entries are mostly still in the ring, where the deep stacks of dense
      // hulls (whose joints are usually convex at once) would have many window entries
      // recomputed from their checkpoints.
      const uint64_t gmk = gsz == kWave ? ~0ull : (((1ull << gsz) - 1ull) << g0);
      settled = !merge || (__ballot(d > kWinDepth) & gmk) != 0;
    }
    const bool serial = merge && (r < kWinRound || settled);
    if (r >= kWinRound && __any(merge && !settled)) {
      // The group's lanes gather the vertices next to s into registers: lane k of the group
      // takes a_{k+1}, the (k+1)-th vertex of A left of s, and b_{k+1}, the (k+1)-th of B right
      // of it (gsz - 1 of each at most), and both walks run there, a ballot for each move.  The
      // positions are those of the serial walk below, which continues from them when a walk
      // leaves its window.
      const int k = lane - g0;
      const uint64_t gm = gsz == kWave ? ~0ull : ((1ull << gsz) - 1ull);
      const bool inA = merge && lane < sB, inB = merge && lane >= sB && lane <= lb;
      const bool ne = lo <= hi;
      const int topA = lane == sB - 1 ? min(hi, d - 2) : hi;  // (s itself is a_0)
      const int cA = (inA && ne) ? max(topA - lo + 1, 0) : 0;
      const int cB = (inB && ne) ? hi - lo + 1 : 0;
      int incl = cA + cB;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += v;
      }
      const int atS = __shfl(incl, sB - 1 < kWave ? sB - 1 : kWave - 1, kWave);
      const int atG0 = __shfl(incl, g0 > 0 ? g0 - 1 : 0, kWave);
      const int atL = __shfl(incl, lb >= 0 ? lb : 0, kWave);
      const int totA = atS - (g0 > 0 ? atG0 : 0), totB = atL - atS;
      const int nA = min(totA + 1, gsz - 1), nB = min(totB, gsz - 1);
      const bool exA = totA + 1 <= gsz - 1, exB = totB <= gsz - 1;
      if (inA) {
        const int sx = atS - incl;  // A's vertices in the lanes right of this one
        for (int m = 0; m < cA && sx + m < nA; ++m) L.wa[g0 + sx + m] = (uint32_t)(lane << 16 | (topA - m));
      }
      if (merge && lane == g0 && totA < nA) L.wa[g0 + totA] = (uint32_t)(g0 << 16);  // (g0, 0): A's first
      if (inB) {
        const int px = incl - cB - atS;  // B's vertices in the lanes left of this one
        for (int m = 0; m < cB && px + m < nB; ++m) L.wb[g0 + px + m] = (uint32_t)(lane << 16 | (lo + m));
      }
      __syncthreads();
      int oal = 0, oad = 0, obl = 0, obd = 0;
      double2 PA{0.0, 0.0}, PB{0.0, 0.0};
      if (merge && !settled && k < nA) {
        const uint32_t e = L.wa[lane];
        oal = (int)(e >> 16);
        oad = (int)(e & 0xffffu);
        PA = chunk_entry<T, W, D>(L, ckx, cky, oal, oad, len, yc, wc);
      }
      if (merge && !settled && k < nB) {
        const uint32_t e = L.wb[lane];
        obl = (int)(e >> 16);
        obd = (int)(e & 0xffffu);
        PB = chunk_entry<T, W, D>(L, ckx, cky, obl, obd, len, yc, wc);
      }
      const int sl = merge ? sB - 1 : 0;
      const int sd = merge ? L.depth[sl] - 1 : 0;
      const double2 Sp = merge ? L.start[sB] : double2{0.0, 0.0};  // s, lane sB - 1's end point
      // lane k: a_k (its left neighbour's a_{k+1}; s for k = 0) and b_{k+2}
      double2 Aprev{__shfl_up(PA.x, 1, kWave), __shfl_up(PA.y, 1, kWave)};
      int apl = __shfl_up(oal, 1, kWave), apd = __shfl_up(oad, 1, kWave);
      if (k == 0) {
        Aprev = Sp;
        apl = sl;
        apd = sd;
      }
      const double2 Bnext{__shfl_down(PB.x, 1, kWave), __shfl_down(PB.y, 1, kWave)};
      const int bnl = __shfl_down(obl, 1, kWave), bnd = __shfl_down(obd, 1, kWave);
      int ka = 0, kb = 1;
      double2 Pa = Sp;
      double2 Pb{__shfl(PB.x, g0, kWave), __shfl(PB.y, g0, kWave)};
      {
        const int b1l = __shfl(obl, g0, kWave), b1d = __shfl(obd, g0, kWave);
        if (!settled) {
          al = sl;
          ai = sd;
          bl = b1l;
          bi = b1d;
        }
      }
      bool act = merge && !settled && nB >= 1;
      for (int it = 0; it < 4 * kWave; ++it) {
        if (!__any(act)) break;
        bool moved = false;
        // alpha: lane k decides the stop at a_k (k = nA: a_nA is A's first vertex when exA)
        {
          const bool st = act && k >= ka &&
                          ((k < nA && wleft(oal, oad, PA, apl, apd, Aprev, bl, bi, Pb)) || (k == nA && exA));
          const uint64_t hit = (__ballot(st) >> g0) & gm;
          const int kk = hit ? __builtin_ctzll(hit) : nA;  // no stop: alpha walks past the window
          const int src = g0 + max(kk - 1, 0);
          const double2 Pn{__shfl(PA.x, src, kWave), __shfl(PA.y, src, kWave)};
          const int nl_ = __shfl(oal, src, kWave), nd_ = __shfl(oad, src, kWave);
          if (act && kk != ka) {
            moved = true;
            ka = kk;
            Pa = kk == 0 ? Sp : Pn;
            al = kk == 0 ? sl : nl_;
            ai = kk == 0 ? sd : nd_;
          }
          if (act && !hit) {
            act = false;
            from_win = true;
          }
        }
        // beta: lane k decides the stop at b_{k+1} (k + 1 = nB: B's last vertex when exB)
        {
          const int k1 = k + 1;
          const bool st = act && k1 >= kb &&
                          ((k1 < nB && wleft(al, ai, Pa, obl, obd, PB, bnl, bnd, Bnext)) || (k1 == nB && exB));
          const uint64_t hit = (__ballot(st) >> g0) & gm;
          const int kk = hit ? __builtin_ctzll(hit) + 1 : nB;
          const int src = g0 + kk - 1;
          const double2 Pn{__shfl(PB.x, src, kWave), __shfl(PB.y, src, kWave)};
          const int nl_ = __shfl(obl, src, kWave), nd_ = __shfl(obd, src, kWave);
          if (act && kk != kb) {
            moved = true;
            kb = kk;
            Pb = Pn;
            bl = nl_;
            bi = nd_;
          }
          if (act && !hit) {
            act = false;
            from_win = true;
          }
        }
        if (act && !moved) {
          act = false;
          settled = true;
        }
      }
      if (merge && !settled) from_win = true;  // (the iteration cap: continue serially)
      __syncthreads();  // (the window slots are rewritten by the next round)
    }
    // a strict left turn of three stack entries: the fast turn of the chunk-relative hi parts
    // when it exceeds its error bound, else the turn of the pairs (wleft above)
    if (merge && lane == sB && (serial || (!settled && from_win))) {
      if (!from_win) {
        al = sB - 1;
        ai = L.depth[al] - 1;                        // alpha = s
        bl = min(__builtin_ctzll(nzr & ~lanes_below(sB)), lb);  // beta = B's first vertex
        bi = L.lo[bl];
      }
      double2 Pa = chunk_entry<T, W, D>(L, ckx, cky, al, ai, len, yc, wc);
      double2 Pb = chunk_entry<T, W, D>(L, ckx, cky, bl, bi, len, yc, wc);
      for (int pass = 0; pass <= kChunk; ++pass) {
        bool moved = false;
        // alpha moves left while (pred alpha, alpha, beta) is not a strict left turn
        while (!(al == g0 && ai == 0)) {
          int pl, pi;
          if (ai > max(L.lo[al], 1)) {
            pl = al;
            pi = ai - 1;
          } else {
            const uint64_t below = nzr & lanes_below(al) & ~lanes_below(g0);
            if (below) {
              pl = 63 - __builtin_clzll(below);
              pi = L.hi[pl];
            } else {
              pl = g0;
              pi = 0;
            }
          }
          const double2 Pp = chunk_entry<T, W, D>(L, ckx, cky, pl, pi, len, yc, wc);
          if (wleft(pl, pi, Pp, al, ai, Pa, bl, bi, Pb)) break;
          al = pl;
          ai = pi;
          Pa = Pp;
          moved = true;
        }
        // beta moves right while (alpha, beta, succ beta) is not a strict left turn
        while (!(bl == lb && bi == L.depth[lb] - 1)) {
          int ql, qi;
          if (bi < L.hi[bl]) {
            ql = bl;
            qi = bi + 1;
          } else {
            ql = min(__builtin_ctzll(nzr & ~lanes_below(bl + 1)), lb);
            qi = max(L.lo[ql], 1);
          }
          const double2 Pq = chunk_entry<T, W, D>(L, ckx, cky, ql, qi, len, yc, wc);
          if (wleft(al, ai, Pa, bl, bi, Pb, ql, qi, Pq)) break;
          bl = ql;
          bi = qi;
          Pb = Pq;
          moved = true;
        }
        if (!moved) break;
      }
    }
    const int src = merge ? sB : lane;
    al = __shfl(al, src, kWave);
    ai = __shfl(ai, src, kWave);
    bl = __shfl(bl, src, kWave);
    bi = __shfl(bi, src, kWave);
    if (merge) {
      if (lane == al) hi = ai;
      if (lane > al && lane < bl) {
        lo = 1;
        hi = 0;
      }
      if (lane == bl) lo = bi;
    }
    L.lo[lane] = lo;
    L.hi[lane] = hi;
    __syncthreads();
  }

  // ---- a5: emit.
  const bool nonempty = lo <= hi;
  const int cnt = (nonempty ? hi - lo + 1 : 0) + (lane == 0 ? 1 : 0);
  int incl = cnt;
#pragma unroll
  for (int dd = 1; dd < kWave; dd <<= 1) {
    const int v = __shfl_up(incl, dd, kWave);
    if (lane >= dd) incl += v;
  }
  const int total = __shfl(incl, kWave - 1, kWave);
  const int rank = incl - cnt;
  const uint32_t fl = (__ballot((f & ISO_ROW_NONFINITE_BIT) != 0) ? ISO_ROW_NONFINITE_BIT : 0u) |
                      (__ballot((f & ISO_ROW_BAD_WEIGHT_BIT) != 0) ? ISO_ROW_BAD_WEIGHT_BIT : 0u);
  const bool listable = total <= kListCap;
  // a chunk with an undecided turn keeps form byte 3 and is processed again by the exact pass
  const bool ilane = frac == 0.0 && (W ? lx : (double)c) < 0x1p25 && aabs < 0x1p25;
  const bool leave = !EXACT && __any(undec && !ilane);
  if (lane == 0) {
    out.nverts[g] = total;
    out.desc[g] = make_int4(j, 0, total - 1, desc_w(listable ? 0 : 1, total));
    out.nseg[g] = 1;
    out.cflags[g] = fl;
    out.dform[g] = leave ? 3 : listable ? 0 : 1;
    const double2 E = L.start[nl], El = L.startl[nl];
    out.tot[g] = make_double2(E.x, E.y);
    out.totl()[g] = make_double2(El.x, El.y);
  }
  if (listable) {
    const int64_t lb0 = g * (int64_t)kListCap;
    int pos = rank;
    if (lane == 0) {
      out.lk[lb0] = 0;
      out.lx[lb0] = 0.0;
      out.ly[lb0] = 0.0;
      out.lxl()[lb0] = 0.0;
      out.lyl()[lb0] = 0.0;
      pos = 1;
    }
    // every lane integral: the chunk's coordinates are integers below 2^31, exact in the hi parts
    const bool exact_chunk = __all(ilane);
    for (int i = lo; i <= hi; ++i) {
      int q;
      PD P;
      if (exact_chunk) {
        const double2 Ph = chunk_entry<T, W, D>(L, ckx, cky, lane, i, len, yc, wc, q);
        P = PD{DD{Ph.x, 0.0}, DD{Ph.y, 0.0}};
      } else {
        P = chunk_entry_dd<T, W, D>(L, ckx, cky, ckxl, ckyl, lane, i, len, yc, wc, q);
      }
      out.lk[lb0 + pos] = (uint16_t)(e0 + q);
      out.lx[lb0 + pos] = P.x.hi;
      out.ly[lb0 + pos] = P.y.hi;
      out.lxl()[lb0 + pos] = P.x.lo;
      out.lyl()[lb0 + pos] = P.y.lo;
      ++pos;
    }
    return;
  }
  // dense form: vertex bits of the chunk's points, set bits before each word, lane starts and
  // checkpoints (coordinates are recomputed from these and the inputs); vertices 1 and V - 2,
  // which the merge levels test at every chunk boundary, are also stored directly.
  {
    const uint64_t nz = __ballot(nonempty);
    const int l1 = __builtin_ctzll(nz);       // vertex 1: the first entry of the first range
    const int lz = 63 - __builtin_clzll(nz);  // vertex V - 1 ends the last range
    if (lane == l1) {
      int q;
      const PD P = chunk_entry_dd<T, W, D>(L, ckx, cky, ckxl, ckyl, lane, lo, len, yc, wc, q);
      out.bnd[g].x = P.x.hi;
      out.bnd[g].y = P.y.hi;
      out.bndl()[g].x = P.x.lo;
      out.bndl()[g].y = P.y.lo;
      out.bndk[g].x = e0 + q;
    }
    // vertex V - 2: the entry before lz's last, or the last of the range before it, or point 0
    const uint64_t before = nz & lanes_below(lz);
    const int lp = before ? 63 - __builtin_clzll(before) : 0;
    const int lzc = __shfl(hi - lo, lz, kWave);   // (entries in lz's range) - 1
    const int src = lzc >= 1 ? lz : lp;
    if (lane == src) {
      const bool in_lz = lzc >= 1;
      int i = in_lz ? hi - 1 : hi;
      PD P{DD{0.0, 0.0}, DD{0.0, 0.0}};
      int kq = 0;
      if (in_lz || before) {
        int q;
        P = chunk_entry_dd<T, W, D>(L, ckx, cky, ckxl, ckyl, lane, i, len, yc, wc, q);
        kq = e0 + q;
      }
      out.bnd[g].z = P.x.hi;
      out.bnd[g].w = P.y.hi;
      out.bndl()[g].z = P.x.lo;
      out.bndl()[g].w = P.y.lo;
      out.bndk[g].y = kq;
    }
  }
  int qlo = kSub + 1, qhi = -1;  // the stack bits of depths lo..hi span points [qlo, qhi]
  if (nonempty) {
    bool in_ring;
    qlo = lane_index<W>(L, lane, lo, c, in_ring);
    qhi = hi == d - 1 ? c : lane_index<W>(L, lane, hi, c, in_ring);
  }
  // bit 0 of the lane's first word is the previous lane's end point
  const int top_kept = (nonempty && hi == d - 1 && c == kSub) ? 1 : 0;
  const int prev_top = __shfl(top_kept, lane > 0 ? lane - 1 : 0, kWave);
  const int64_t mb = g * (int64_t)kMaskW;
  uint32_t words[kLaneW];
  int pc = 0;
#pragma unroll
  for (int wd = 0; wd < kLaneW; ++wd) {
    uint32_t v = L.smask[wd][lane];
    const int a = qlo - kCk * wd, b = qhi - kCk * wd;  // keep bits a..b
    uint32_t keep = 0u;
    if (b >= 0 && a <= 31) {
      const int a2 = max(a, 0), b2 = min(b, 31);
      keep = (b2 >= 31 ? 0xffffffffu : ((2u << b2) - 1u)) & ~((1u << a2) - 1u);
    }
    v &= keep;
    if (wd == 0) v = (v & ~1u) | (lane == 0 ? 1u : (uint32_t)prev_top);
    words[wd] = v;
    pc += __popc(v);
  }
  int wincl = pc;
#pragma unroll
  for (int dd = 1; dd < kWave; dd <<= 1) {
    const int v = __shfl_up(wincl, dd, kWave);
    if (lane >= dd) wincl += v;
  }
  int run = wincl - pc;
#pragma unroll
  for (int wd = 0; wd < kLaneW; ++wd) {
    out.mask[mb + kLaneW * lane + wd] = words[wd];
    out.mcnt[mb + kLaneW * lane + wd] = (uint16_t)run;
    run += __popc(words[wd]);
  }
  if (lane == kWave - 1) {
    out.mask[mb + kMaskW - 1] = (len == kChunk) ? (uint32_t)top_kept : 0u;
    out.mcnt[mb + kMaskW - 1] = (uint16_t)run;
  }
  const int64_t sb = g * (int64_t)kWave;
  if (W) {
    out.lsx[sb + lane] = L.start[lane].x;
    out.lsxl()[sb + lane] = L.startl[lane].x;
  }
  out.lsy[sb + lane] = L.start[lane].y;
  out.lsyl()[sb + lane] = L.startl[lane].y;
}

}  // namespace iso
