// iso_merge.h -- the levels of the segment-list merge tree, one wavefront per merge (gfx950).
//
// "Merge Hulls Without Copying Vertices: GPU Isotonic Regression":
//   Section 3.3 / Definition 4.3 / Theorem 4.4  a node's hull is a list of segments (chunk,
//                first, last) of chunk hulls, stored in the descriptor slots of its chunks; a merge
//                cuts one segment of each child and moves the right child's tail down.
//   Lemma 4.2    the bridge is found by walking from the shared point s: alpha moves left while
//                (pred alpha, alpha, beta) is not a strict left turn, beta right symmetrically,
//                until neither moves (alpha the leftmost, beta the rightmost contact).
//   Section 5.2  a walk that runs long is replaced by a search (here the Overmars-van Leeuwen
//                bisection of iso_geom.h).
//
// On the page a level runs one thread per merge when it has many merges, one launch per level.
// Here every merge has a wavefront, and one launch takes three levels: a workgroup of four
// wavefronts merges a subtree of eight nodes (four merges, then two, then one, with a barrier
// between levels), so a row of m chunks needs ceil(log2 m / 3) launches.  It first reads up to 64 list-form vertices on each side of s into registers and
// runs both walks there, one ballot per walk (window_bridge); that settles nearly every merge
// of the lower levels.  A longer walk continues in memory 256 vertices at a time: the lanes
// gather the next vertices of the walk (the segments' lengths come from one coalesced read of
// descriptors and a scan), test the walk's predicate on all of them at once and take the first
// stop with a ballot.  Where s lies in a dense-form chunk, a few single steps come first, since a
// dense hull's bridge is usually a vertex or two from s.  The tail of the right child's list is
// moved by all lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "iso_geom.h"

namespace iso {

constexpr int kMergeWaves = 4;   // merges per workgroup of 256

struct MergeLds {
  int cum[kWave];
  Desc d[kWave];
};

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ GPt shfl_up_pt(const GPt& p, int lane) {
  GPt r;
  r.x = __shfl_up(p.x, 1, kWave);
  r.y = __shfl_up(p.y, 1, kWave);
  r.sxh = __shfl_up(p.sxh, 1, kWave);
  r.sxl = __shfl_up(p.sxl, 1, kWave);
  r.syh = __shfl_up(p.syh, 1, kWave);
  r.syl = __shfl_up(p.syl, 1, kWave);
  (void)lane;
  return r;
}

__device__ __forceinline__ GPt shfl_pt(const GPt& p, int src) {
  GPt r;
  r.x = __shfl(p.x, src, kWave);
  r.y = __shfl(p.y, src, kWave);
  r.sxh = __shfl(p.sxh, src, kWave);
  r.sxl = __shfl(p.sxl, src, kWave);
  r.syh = __shfl(p.syh, src, kWave);
  r.syl = __shfl(p.syl, src, kWave);
  return r;
}

// One window of a walk over the list L from v (exclusive), in direction dir (-1: towards the
// list's first vertex, +1: towards its last): the kWalkK * kWave vertices after v, lane i taking
// v_{kWalkK i + 1} .. v_{kWalkK i + kWalkK}.  The segments' lengths come from one read of up to
// kWalkK * kWave descriptors and a scan in LDS.  The walk stops at v_i when stop(v_i, v_{i+1})
// holds; returns true when it stopped inside this window, and in every case advances v and Pv to
// where the walk stands.
constexpr int kWalkK = 4;
constexpr int kWideCap = 32;  // wide windows of one side pass before switching to the search
constexpr int kShortWalk = 8;  // single steps tried before memory windows at dense joints

struct WideLds {
  int cum[kWalkK * kWave];
  Desc d[kWalkK * kWave];
};

template <class VS, class Stop>
__device__ __forceinline__ bool walk_window_wide(const VS& S, const NodeList& L, int dir, VRef& v, GPt& Pv,
                                 int lane, WideLds& W, Stop stop) {
  constexpr int NW = kWalkK * kWave;
  // segments j = lane * kWalkK + t: v.u + dir * j, and the number of their vertices beyond v
  int cnt[kWalkK];
  int lsum = 0;
#pragma unroll
  for (int t = 0; t < kWalkK; ++t) {
    const int jj = lane * kWalkK + t;
    const int uj = v.u + dir * jj;
    Desc dj = make_int4(0, 0, -1, 0);
    int c = 0;
    if (uj >= 0 && uj < L.n) {
      dj = L.d[uj];
      if (jj == 0) c = dir < 0 ? v.p - dj.y : dj.z - v.p;
      else c = dj.z - dj.y + 1;
    }
    W.d[jj] = dj;
    cnt[t] = c;
    lsum += c;
  }
  int incl = lsum;
#pragma unroll
  for (int dd = 1; dd < kWave; dd <<= 1) {
    const int o = __shfl_up(incl, dd, kWave);
    if (lane >= dd) incl += o;
  }
  int run = incl - lsum;
#pragma unroll
  for (int t = 0; t < kWalkK; ++t) {
    run += cnt[t];
    W.cum[lane * kWalkK + t] = run;
  }
  wave_sync();
  const int total = __shfl(incl, kWave - 1, kWave);
  VRef mine[kWalkK];
  GPt P[kWalkK];
  bool valid[kWalkK];
  // the segment of each of this lane's vertices: the number of segments whose cumulative count is
  // below the vertex's ordinal, by strides over the power-of-two table (the kWalkK searches run
  // side by side)
  static_assert((NW & (NW - 1)) == 0, "stride search");
  int seg[kWalkK];
#pragma unroll
  for (int t = 0; t < kWalkK; ++t) seg[t] = 0;
#pragma unroll
  for (int st = NW / 2; st > 0; st >>= 1) {
#pragma unroll
    for (int t = 0; t < kWalkK; ++t) {
      const int want = lane * kWalkK + t + 1;
      if (W.cum[seg[t] + st - 1] < want) seg[t] += st;
    }
  }
#pragma unroll
  for (int t = 0; t < kWalkK; ++t) {
    const int want = lane * kWalkK + t + 1;
    valid[t] = want <= total;
    mine[t] = v;
    P[t] = Pv;
    if (valid[t]) {
      const int lo = seg[t];
      const int before = lo > 0 ? W.cum[lo - 1] : 0;
      const int k = want - before - 1;
      const Desc d = W.d[lo];
      int rank;
      if (dir < 0) rank = (lo == 0) ? v.p - 1 - k : d.z - k;
      else rank = (lo == 0) ? v.p + 1 + k : d.y + k;
      mine[t] = VRef{v.u + dir * lo, rank};
      P[t] = S.pt_desc(L.row, d, rank);
    }
  }
  wave_sync();
  // v_{K i} (the vertex before this lane's first): the previous lane's last, lane 0: v
  GPt Pi = shfl_up_pt(P[kWalkK - 1], lane);
  if (lane == 0) Pi = Pv;
  int first = kWalkK;  // this lane's first stop or run-out (t: stop between v_{K i + t} and v_{K i + t + 1})
  bool first_stop = false;
#pragma unroll
  for (int t = kWalkK - 1; t >= 0; --t) {
    const GPt& a = t == 0 ? Pi : P[t - 1];
    const bool st = valid[t] && stop(a, P[t]);
    if (st || !valid[t]) {
      first = t;
      first_stop = st;
    }
  }
  const uint64_t hit = __ballot(first < kWalkK);
  const int fl = hit ? __builtin_ctzll(hit) : kWave;
  int f = NW;  // walk position reached: v_f
  bool stop_at_f = false;
  if (fl < kWave) {
    f = fl * kWalkK + __shfl(first, fl, kWave);
    stop_at_f = __shfl(first_stop ? 1 : 0, fl, kWave) != 0;
  }
  const bool list_end = (dir < 0) ? (v.u - (NW - 1) <= 0) : (v.u + (NW - 1) >= L.n - 1);
  if (f > 0) {
    // v_f is vertex f - 1 of the window: lane (f - 1) / K, slot (f - 1) % K
    const int src = (f - 1) / kWalkK, slot = (f - 1) % kWalkK;
    VRef mr = mine[0];
    GPt mp = P[0];
#pragma unroll
    for (int t = 1; t < kWalkK; ++t)
      if (slot == t) {
        mr = mine[t];
        mp = P[t];
      }
    v = VRef{__shfl(mr.u, src, kWave), __shfl(mr.p, src, kWave)};
    Pv = shfl_pt(mp, src);
  }
  return stop_at_f || (f < NW && list_end);
}

// Walk to the bridge one vertex at a time, from alpha in A and beta in B, for at most `steps`
// moves (steps < 0: no cap).  Returns true when the walk ends (a round in which neither side
// moves), false with the positions reached when the moves run out.  Every lane walks the same
// vertices.
template <class VS>
__device__ __forceinline__ bool merge_finish_walk(const VS& S, const NodeList& LA, const NodeList& LB, VRef firstA,
                                  VRef lastB, VRef& al, VRef& be, int steps) {
  GPt Pa = load_v(S, LA, al), Pb = load_v(S, LB, be);
  for (;;) {
    bool moved = false;
    while (!vref_eq(al, firstA)) {
      const VRef p = list_pred(LA, al);
      const GPt Pp = load_v(S, LA, p);
      if (gleft(Pp, Pa, Pb)) break;
      if (steps == 0) return false;
      --steps;
      al = p;
      Pa = Pp;
      moved = true;
    }
    while (!vref_eq(be, lastB)) {
      const VRef q = list_succ(LB, be);
      const GPt Pq = load_v(S, LB, q);
      if (gleft(Pa, Pb, Pq)) break;
      if (steps == 0) return false;
      --steps;
      be = q;
      Pb = Pq;
      moved = true;
    }
    if (!moved) return true;
  }
}

// The vertices beyond s on each side of a merge, up to kWave - 1 of them, stopping before the
// first dense-form segment: lane i gets v_{i+1}, the (i+1)-th vertex from s (mine, P), towards
// A's first vertex from sA and towards B's last from sB; n: how many, ex: the window reaches the
// end of the list.  Both sides are read together, so that their memory and LDS round trips
// overlap: one read of descriptors, a scan, one wavefront sync, side-by-side searches, one read of
// points.
template <class VS>
__device__ __forceinline__ void side_windows2(const VS& S, const NodeList& LA, VRef sA, const NodeList& LB,
                                              VRef sB, int lane, MergeLds& WA, MergeLds& WB, int& na,
                                              bool& exA, VRef& mineA, GPt& PA, int& nb, bool& exB,
                                              VRef& mineB, GPt& PB, GPt& Ps) {
  const int uA = sA.u - lane, uB = sB.u + lane;
  const bool inA = uA >= 0, inB = uB < LB.n;
  Desc dA = make_int4(0, 0, -1, 0), dB = make_int4(0, 0, -1, 0);
  if (inA) dA = LA.d[uA];
  if (inB) dB = LB.d[uB];
  // s itself (vertex sA.p of A's last segment), read while the windows are located
  Ps = S.pt_desc(LA.row, LA.d[sA.u], sA.p);
  const uint64_t dmA = __ballot(inA && desc_form(dA) != 0), dmB = __ballot(inB && desc_form(dB) != 0);
  const int fdA = dmA ? __builtin_ctzll(dmA) : kWave, fdB = dmB ? __builtin_ctzll(dmB) : kWave;
  int cA = 0, cB = 0;
  if (inA && lane < fdA) cA = lane == 0 ? sA.p - dA.y : dA.z - dA.y + 1;
  if (inB && lane < fdB) cB = lane == 0 ? dB.z - sB.p : dB.z - dB.y + 1;
  int cumA = cA, cumB = cB;
#pragma unroll
  for (int dd = 1; dd < kWave; dd <<= 1) {
    const int oA = __shfl_up(cumA, dd, kWave), oB = __shfl_up(cumB, dd, kWave);
    if (lane >= dd) {
      cumA += oA;
      cumB += oB;
    }
  }
  WA.cum[lane] = cumA;
  WA.d[lane] = dA;
  WB.cum[lane] = cumB;
  WB.d[lane] = dB;
  wave_sync();
  const int totA = __shfl(cumA, kWave - 1, kWave), totB = __shfl(cumB, kWave - 1, kWave);
  na = min(totA, kWave - 1);
  nb = min(totB, kWave - 1);
  exA = fdA == kWave && (sA.u - (kWave - 1) <= 0) && totA <= kWave - 1;
  exB = fdB == kWave && (sB.u + (kWave - 1) >= LB.n - 1) && totB <= kWave - 1;
  mineA = sA;
  mineB = sB;
  PA = GPt{0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  PB = PA;
  const int want = lane + 1;
  // smallest j with cum[j] >= want, on both tables side by side
  int loA = 0, hiA = kWave - 1, loB = 0, hiB = kWave - 1;
#pragma unroll
  for (int st = 0; st < 6; ++st) {
    const int midA = (loA + hiA) >> 1, midB = (loB + hiB) >> 1;
    const int vA = WA.cum[midA], vB = WB.cum[midB];
    if (loA < hiA) {
      if (vA >= want) hiA = midA;
      else loA = midA + 1;
    }
    if (loB < hiB) {
      if (vB >= want) hiB = midB;
      else loB = midB + 1;
    }
  }
  if (want <= na) {
    const int before = loA > 0 ? WA.cum[loA - 1] : 0;
    const int k = want - before - 1;
    const Desc d = WA.d[loA];
    const int rank = (loA == 0) ? sA.p - 1 - k : d.z - k;
    mineA = VRef{sA.u - loA, rank};
    PA = S.pt_list(LA.row, d.x, rank);
  }
  if (want <= nb) {
    const int before = loB > 0 ? WB.cum[loB - 1] : 0;
    const int k = want - before - 1;
    const Desc d = WB.d[loB];
    const int rank = (loB == 0) ? sB.p + 1 + k : d.y + k;
    mineB = VRef{sB.u + loB, rank};
    PB = S.pt_list(LB.row, d.x, rank);
  }
}

// First phase of a merge: the walk of Lemma 4.2 on the vertices next to s.  Both side windows are
// read at once (a_i = the i-th vertex of A left of s, b_i of B right of s, a_0 = b_0 = s), then
// the walks alternate on registers: alpha stops at a_k when (a_{k+1}, a_k, beta) is a strict
// left turn, beta at b_k when (alpha, b_k, b_{k+1}) is; each walk's first stop is found with a
// ballot.  Returns true with the bridge (al, be) when both walks end inside their windows, else
// false with the furthest positions reached (al, be, Pa, Pb), from which the walk continues in
// memory.
template <class VS>
__device__ __forceinline__ bool window_bridge(const VS& S, const NodeList& LA, const NodeList& LB, int lane,
                              MergeLds& WA, MergeLds& WB, GPt& Sp, VRef& al, VRef& be,
                              GPt& Pa, GPt& Pb) {
  int na, nb;
  bool exA, exB;
  VRef ra, rb;
  GPt PA, PB;
  side_windows2(S, LA, list_last(LA), LB, list_first(LB), lane, WA, WB, na, exA, ra, PA, nb, exB, rb, PB, Sp);
  al = list_last(LA);
  Pa = Sp;
  if (nb < 1) {  // (no list-form vertex after s in B's window)
    be = list_succ(LB, list_first(LB));
    Pb = load_v(S, LB, be);
    return false;
  }
  be = VRef{__shfl(rb.u, 0, kWave), __shfl(rb.p, 0, kWave)};
  Pb = shfl_pt(PB, 0);
  int ka = 0, kb = 1;
  const GPt Aprev = [&]() {  // lane i: a_i
    GPt r = shfl_up_pt(PA, lane);
    if (lane == 0) r = Sp;
    return r;
  }();
  const GPt Bnext = [&]() {  // lane i: b_{i+2}
    GPt r;
    r.x = __shfl_down(PB.x, 1, kWave);
    r.y = __shfl_down(PB.y, 1, kWave);
    r.sxh = __shfl_down(PB.sxh, 1, kWave);
    r.sxl = __shfl_down(PB.sxl, 1, kWave);
    r.syh = __shfl_down(PB.syh, 1, kWave);
    r.syl = __shfl_down(PB.syl, 1, kWave);
    return r;
  }();
  for (int it = 0; it < 4 * kWave; ++it) {
    bool moved = false;
    // alpha: lane i decides k = i (a_{i+1} = its own PA); k = na has no a_{na+1} in the window
    {
      const bool st = lane >= ka && ((lane < na && gleft(PA, Aprev, Pb)) || (lane == na && exA));
      const uint64_t hit = __ballot(st);
      if (!hit) {  // alpha walks past the window
        ka = na;
        al = ka == 0 ? list_last(LA) : VRef{__shfl(ra.u, ka - 1, kWave), __shfl(ra.p, ka - 1, kWave)};
        if (ka > 0) Pa = shfl_pt(PA, ka - 1);
        return false;
      }
      const int k = __builtin_ctzll(hit);
      if (k != ka) {
        moved = true;
        ka = k;
        al = VRef{__shfl(ra.u, ka - 1, kWave), __shfl(ra.p, ka - 1, kWave)};
        Pa = shfl_pt(PA, ka - 1);
      }
    }
    // beta: lane i decides k = i + 1 (b_{i+1} = its own PB, b_{i+2} from lane i + 1); k = nb
    // has no b_{nb+1} in the window
    {
      const int k1 = lane + 1;
      const bool st = k1 >= kb && ((k1 < nb && gleft(Pa, PB, Bnext)) || (k1 == nb && exB));
      const uint64_t hit = __ballot(st);
      if (!hit) {  // beta walks past the window
        kb = nb;
        be = VRef{__shfl(rb.u, kb - 1, kWave), __shfl(rb.p, kb - 1, kWave)};
        Pb = shfl_pt(PB, kb - 1);
        return false;
      }
      const int k = __builtin_ctzll(hit) + 1;
      if (k != kb) {
        moved = true;
        kb = k;
        be = VRef{__shfl(rb.u, kb - 1, kWave), __shfl(rb.p, kb - 1, kWave)};
        Pb = shfl_pt(PB, kb - 1);
      }
    }
    if (!moved) return true;
  }
  return false;
}

// Merges node A (chunks from jA) with node B (chunks from jB) of one row: one wavefront.
template <typename T, bool W, bool D>
__device__ __forceinline__ void merge_pair(const VertexStore<T, W, D>& S, int64_t row, int jA, int jB,
                                           int lane, MergeLds& WA, MergeLds& WB, WideLds& Ww) {
  const int64_t rb = row * S.m;
  Desc* dA = S.desc + rb + jA;
  Desc* dB = S.desc + rb + jB;
  const NodeList LA{dA, S.nseg[rb + jA], row};
  const NodeList LB{dB, S.nseg[rb + jB], row};
  const VRef firstA = list_first(LA);
  const VRef lastB = list_last(LB);
  VRef al, be;
  GPt Pa, Pb;
  GPt Sp;  // the shared point s, A's last vertex (read by window_bridge)
  bool settled = window_bridge(S, LA, LB, lane, WA, WB, Sp, al, be, Pa, Pb);
  if (!settled) {
    // both walks may already stop where the windows ended (always the case at a strictly convex
    // s, which dense-form chunks, outside the windows, reach this way): one step of each side
    settled = true;
    if (!vref_eq(al, firstA)) {
      const GPt Pp = load_v(S, LA, list_pred(LA, al));
      if (!(gleft(Pp, Pa, Pb))) settled = false;
    }
    if (settled && !vref_eq(be, lastB)) {
      // (alpha, beta, succ beta) three consecutive points of a chunk whose y is strictly
      // increasing (form 2: vertices are points) turn strictly left in exact arithmetic, the
      // slopes of the two one-element edges being consecutive y values
      const Desc d0 = LB.d[0];
      const bool consecutive = desc_form(d0) == 2 && be.u == 0 && vref_eq(al, list_last(LA)) &&
                               be.p == d0.y + 1 && be.p < d0.z;
      if (!consecutive) {
        const GPt Pq = load_v(S, LB, list_succ(LB, be));
        if (!(gleft(Pa, Pb, Pq))) settled = false;
      }
    }
  }
  // What is left is walked in phases: 0, a few single steps (taken first when s lies in a
  // dense-form chunk on one side, where the bridge is usually a vertex or two from s and a single
  // step reads one vertex where a memory window recomputes 256 of them); 1, memory windows, then
  // the Overmars-van Leeuwen bisection for long walks; 2, single steps to the end (when rounding
  // defeats the bisection).  The single-step walk has one call site, so it stays inline.
  int phase = (desc_form(LA.d[LA.n - 1]) != 0 || desc_form(LB.d[0]) != 0) ? 0 : 1;
  while (!settled) {
    if (phase != 1) {
      settled = merge_finish_walk(S, LA, LB, firstA, lastB, al, be, phase == 0 ? kShortWalk : -1);
      if (!settled) {  // (after phase 0 only: phase 2 always ends)
        Pa = load_v(S, LA, al);
        Pb = load_v(S, LB, be);
        phase = 1;
      }
      continue;
    }
    // the walk continues in memory, kWalkK * 64 vertices at a time, from where it stands
    if (lane == 0) atomicAdd(&g_branch_counts[3], 1ull);
    bool searched = false;
    for (int pass = 0; pass < 4 * kChunk; ++pass) {
      bool moved = false;
      // (from the second pass on, a side whose first step already stops gathers no window)
      bool walk_a = !vref_eq(al, firstA);
      if (pass > 0 && walk_a) walk_a = !(gleft(load_v(S, LA, list_pred(LA, al)), Pa, Pb));
      // A side: alpha moves left while (pred alpha, alpha, beta) is not a strict left turn
      for (int win = 0; walk_a && !vref_eq(al, firstA); ++win) {
        if (win == kWideCap) {
          searched = true;
          break;
        }
        const VRef before = al;
        const bool done = walk_window_wide(S, LA, -1, al, Pa, lane, Ww,
                                           [&](const GPt& vi, const GPt& vn) { return gleft(vn, vi, Pb); });
        if (!vref_eq(before, al)) moved = true;
        if (done) break;
      }
      if (searched) break;
      bool walk_b = !vref_eq(be, lastB);
      if (pass > 0 && walk_b) walk_b = !(gleft(Pa, Pb, load_v(S, LB, list_succ(LB, be))));
      // B side: beta moves right while (alpha, beta, succ beta) is not a strict left turn
      for (int win = 0; walk_b && !vref_eq(be, lastB); ++win) {
        if (win == kWideCap) {
          searched = true;
          break;
        }
        const VRef before = be;
        const bool done = walk_window_wide(S, LB, +1, be, Pb, lane, Ww,
                                           [&](const GPt& vi, const GPt& vn) { return gleft(Pa, vi, vn); });
        if (!vref_eq(before, be)) moved = true;
        if (done) break;
      }
      if (searched || !moved) break;
    }
    settled = true;
    if (searched) {
      // long walk: Overmars-van Leeuwen bisection over the ranges still open (every lane runs the
      // same serial search, reading the same addresses)
      VRef a2, b2;
      if (lane == 0) atomicAdd(&g_branch_counts[0], 1ull);
      if (bridge_search(S, LA, LB, firstA, al, be, lastB, Sp, a2, b2)) {
        al = a2;
        be = b2;
      } else {
        settled = false;  // rounding defeated the search: finish by single steps
        phase = 2;
        if (lane == 0) atomicAdd(&g_branch_counts[1], 1ull);
      }
    }
  }
  // Cut: A keeps segments 0..al.u with the last one ending at al.p; B keeps be.u.. with the first
  // starting at be.p, moved down to follow A's kept part.
  const int nA = al.u + 1;
  const int nB = LB.n - be.u;
  Desc first = dB[be.u];
  first.y = be.p;
  wave_sync();
  if (lane == 0) {
    dA[al.u].z = al.p;
    dA[nA] = first;
  }
  // dA + nA <= dB + be.u, so a write never lands on a descriptor a later read needs; each lane
  // keeps four reads in flight.  When they are equal the tail is already in place.
  constexpr int kCopy = 4;
  const int bstart = (dA + nA == dB + be.u) ? nB : 1;
  for (int b = bstart; b < nB; b += kCopy * kWave) {
    Desc dd[kCopy];
#pragma unroll
    for (int k = 0; k < kCopy; ++k) {
      const int tt = b + k * kWave + lane;
      if (tt < nB) dd[k] = dB[be.u + tt];
    }
#pragma unroll
    for (int k = 0; k < kCopy; ++k) {
      const int tt = b + k * kWave + lane;
      if (tt < nB) dA[nA + tt] = dd[k];
    }
  }
  if (lane == 0) S.nseg[rb + jA] = nA + nB;
}

// Levels r0 .. r0 + nlev - 1 of the merge tree in one launch (nlev <= kMergeGroup): a workgroup
// takes the subtree over 2^(r0 + nlev) chunks of one row and merges it level by level, its
// wavefronts separated by a barrier between levels.  A merge reads only its two children's lists
// (and the chunk hulls, which no merge writes), so subtrees are independent; per_row = subtrees
// per row.
constexpr int kMergeGroup = 3;  // 2^(kMergeGroup - 1) = kMergeWaves merges at the group's first level
static_assert((1 << (kMergeGroup - 1)) <= kMergeWaves, "a group's first level needs a wavefront per merge");
template <typename T, bool W, bool D>
__global__ __launch_bounds__(kMergeWaves * kWave) void k_merge_levels(VertexStore<T, W, D> S, int r0,
                                                                      int nlev, int64_t per_row) {
  __shared__ MergeLds sw[kMergeWaves][2];
  __shared__ WideLds sww[kMergeWaves];
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x / per_row;
  const int64_t sub = (int64_t)blockIdx.x - row * per_row;
  for (int k = 0; k < nlev; ++k) {
    const int r = r0 + k;
    const int nm = 1 << (nlev - 1 - k);  // merges of the subtree at level r
    if (wid < nm) {
      const int64_t jA = (sub * nm + wid) << (r + 1);
      const int64_t jB = jA + ((int64_t)1 << r);
      if (jB < S.m) merge_pair(S, row, (int)jA, (int)jB, lane, sw[wid][0], sw[wid][1], sww[wid]);
    }
    __syncthreads();
  }
}

}  // namespace iso
