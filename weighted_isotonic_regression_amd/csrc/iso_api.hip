// iso_api.hip -- the C ABI of include/iso.h: argument checks, workspace layout and launches.
//
// Paths (by row length n; "Merge Hulls Without Copying Vertices", Section 3 and 6):
//   n <= 16     four lanes per row, pool adjacent violators in registers and LDS (k_tiny)
//   n <= 4096   one row per workgroup of 1024 threads, its diagram in LDS, merged level by level
//               with candidate-parallel bridge searches (k_row, iso_row.h); rows of at most 2048
//               in batches of more than 256 instead packed L = 1, 2, ..., 64 lanes per row,
//               64 / L rows per wavefront (k_wave).  Either launch writes z, block starts and
//               row flags (Section 3.5).
//   n >  4096   rows split into chunks of 16384 (one wavefront each, 256 points per lane):
//               k_increasing (chunks whose diagram is its own hull), k_chunk (chunk hulls; a
//               second, exact instantiation takes the chunks whose fast turns left one undecided),
//               k_scan_reduce + k_scan_apply (chunk starts; k_scan_apply alone for rows of at
//               most 1024 chunks),
//               ceil(ceil(log2 m) / 3) launches of k_merge_levels, k_ends, k_fit
//               (Section 3.3 and 3.4).
// Rows of unequal lengths (iso_fit_ragged) are bucketed by length, padded into a rectangular
// buffer per bucket (iso_ragged.h) and fitted by the paths above.  The soft rank (iso_soft_rank,
// iso_softrank.h) sorts each row with rocPRIM's radix sort and fits the decreasing direction.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include <rocprim/device/device_radix_sort.hpp>
#include <rocprim/iterator/counting_iterator.hpp>

#include "../../include/iso.h"
#include "../../include/iso_profile.h"
#include "iso_kernels.h"
#include "iso_chunk.h"
#include "iso_merge.h"
#include "iso_ragged.h"
#include "iso_row.h"
#include "iso_softrank.h"

// The fixed scratch of iso_fit_noalloc: one copy on every GPU the library runs on, kept until the
// process ends.  Host code never uses this name as an address; scratch_address() looks up the
// copy of the current device once and keeps it.
static __device__ __align__(256) char scratch[ISO_NOALLOC_SCRATCH_BYTES];

static_assert(iso::ISO_ROW_NONFINITE_BIT == ISO_ROW_NONFINITE, "flag bits");
static_assert(iso::ISO_ROW_BAD_WEIGHT_BIT == ISO_ROW_BAD_WEIGHT, "flag bits");

namespace {

using namespace iso;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  size_t total = 0;
  size_t o_rflags = 0, o_any = 0;
  // long rows only
  // arrays of coordinate pairs hold the hi parts of all G chunks, then the lo parts
  size_t o_tot = 0, o_start = 0, o_nv = 0, o_cf = 0, o_desc = 0, o_nseg = 0, o_lk = 0, o_lx = 0,
         o_ly = 0, o_mask = 0, o_mcnt = 0, o_lsx = 0, o_lsy = 0, o_ckx = 0, o_cky = 0, o_zt = 0,
         o_df = 0, o_bnd = 0, o_bndk = 0, o_ends = 0, o_bsum = 0, o_bflag = 0;
  int64_t m = 0, nblk = 0;
};

bool long_rows(int64_t n) { return n > kShortMax; }

Layout make_layout(int64_t batch, int64_t n) {
  Layout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.o_rflags = take((size_t)batch * sizeof(uint32_t));
  L.o_any = take(sizeof(uint32_t));
  if (long_rows(n)) {
    L.m = (n + kChunk - 1) / kChunk;
    L.nblk = (L.m + kScanBlock - 1) / kScanBlock;
    const size_t G = (size_t)batch * (size_t)L.m;
    L.o_tot = take(2 * G * sizeof(double2));
    L.o_start = take(G * sizeof(double4));
    L.o_nv = take(G * sizeof(int));
    L.o_cf = take(G * sizeof(uint32_t));
    L.o_desc = take(G * sizeof(Desc));
    L.o_nseg = take(G * sizeof(int));
    L.o_lk = take(G * (size_t)kListCap * sizeof(uint16_t));
    L.o_lx = take(2 * G * (size_t)kListCap * sizeof(double));
    L.o_ly = take(2 * G * (size_t)kListCap * sizeof(double));
    L.o_mask = take(G * (size_t)kMaskW * sizeof(uint32_t));
    L.o_mcnt = take(G * (size_t)kMaskW * sizeof(uint16_t));
    L.o_lsx = take(2 * G * (size_t)kWave * sizeof(double));
    L.o_lsy = take(2 * G * (size_t)kWave * sizeof(double));
    L.o_ckx = take(2 * G * (size_t)kWave * kLaneW * sizeof(double));
    L.o_cky = take(2 * G * (size_t)kWave * kLaneW * sizeof(double));
    L.o_zt = take(G * (size_t)kWave * sizeof(uint32_t));
    L.o_df = take(G);
    L.o_bnd = take(2 * G * sizeof(double4));
    L.o_bndk = take(G * sizeof(int2));
    L.o_ends = take(G * sizeof(EndInfo));
    L.o_bsum = take((size_t)batch * (size_t)L.nblk * sizeof(double4));
    L.o_bflag = take((size_t)batch * (size_t)L.nblk * sizeof(uint32_t));
  }
  L.total = off;
  return L;
}

bool shape_ok(int64_t batch, int64_t n, int dtype) {
  if (batch < 0 || n < 0) return false;
  if (dtype != ISO_F32 && dtype != ISO_F64) return false;
  if (batch > 0 && n > INT64_MAX / 16 / batch) return false;  // element and byte counts fit
  if (long_rows(n)) {
    const int64_t m = (n + kChunk - 1) / kChunk;
    if (batch > 0 && m > (int64_t)INT32_MAX / batch) return false;  // one launch block per chunk
  } else if (batch > (int64_t)INT32_MAX) {
    return false;
  }
  return true;
}

bool overlaps(const void* a, size_t abytes, const void* b, size_t bbytes) {
  if (!a || !b || abytes == 0 || bbytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + bbytes && b0 < a0 + abytes;
}

// ---- per-stage event timing (iso_profile.h)
struct ProfCall {
  hipEvent_t ev[ISO_PROF_STAGES + 1];
  bool own[ISO_PROF_STAGES + 1];  // false: the previous boundary's event, reused
  int launches[ISO_PROF_STAGES];
  int marks;
};
bool g_prof_on = false;
std::vector<ProfCall> g_prof_calls;

// Records an event before the first kernel and after each stage of one call.
struct Prof {
  bool on;
  hipStream_t s;
  ProfCall c;
  explicit Prof(hipStream_t st) : on(g_prof_on), s(st) {
    c.marks = 0;
    for (int k = 0; k < ISO_PROF_STAGES; ++k) c.launches[k] = 0;
    if (on) mark(0);
  }
  void mark(int launches) {
    if (!on) return;
    if (c.marks > 0) c.launches[c.marks - 1] = launches;
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) {
      on = false;
      return;
    }
    if (hipEventRecord(e, s) != hipSuccess) {
      (void)hipEventDestroy(e);
      on = false;
      return;
    }
    c.own[c.marks] = true;
    c.ev[c.marks++] = e;
  }
  // a stage that launches nothing: its end is its start
  void skip() {
    if (!on || c.marks == 0) return;
    c.launches[c.marks - 1] = 0;
    c.own[c.marks] = false;
    c.ev[c.marks] = c.ev[c.marks - 1];
    ++c.marks;
  }
  ~Prof() {
    if (on && c.marks > 1) g_prof_calls.push_back(c);
  }
};

// ---- scratch of iso_fit_noalloc: its device address, per device, looked up on first use
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(hipStream_t s, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ISO_EHIP;
  if (s) {
    int sdev = -1;
    if (hipStreamGetDevice(s, &sdev) != hipSuccess) return ISO_EHIP;
    if (sdev != dev) return ISO_EINVAL;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ISO_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ISO_OK;
}

// Rows of 2049 to 4096 elements go one to a workgroup of 1024 threads (k_row), where a thread's
// chain is four points long and the merges search their bridges with many threads at once; so do
// shorter rows in batches of at most kRowBatch, which k_row finishes in one round of workgroups
// (256 CUs) in less time than one k_wave wavefront takes.  Larger batches of shorter rows pack
// 64 / L rows per k_wave wavefront.
constexpr int64_t kRowBatch = 256;
bool row_kernel(int64_t batch, int64_t n) { return n > kShortMax / 2 || batch <= kRowBatch; }

int lanes_per_row(int64_t n) {
  int need = (int)((n + kLanePts - 1) / kLanePts);
  int L = 1;
  while (L < need) L <<= 1;
  return L;
}

template <typename T, bool W, bool D>
int run_fit(const T* y, const T* w, T* z, uint8_t* bstart, uint32_t* rflags, int64_t batch,
            int64_t n, char* ws, const Layout& Lay, hipStream_t s, bool row_walk = false) {
  Prof prof(s);
  if (n <= kTinyMax) {
    prof.skip();
    hipLaunchKernelGGL((k_tiny<T, W, D>), dim3((unsigned)((batch + kTinyRows - 1) / kTinyRows)), dim3(kWave), 0, s, y, w, z,
                       bstart, rflags, batch, (int)n);
    prof.mark(1);
    return hipGetLastError() == hipSuccess ? ISO_OK : ISO_EHIP;
  }
  if (!long_rows(n)) {
    const int L = lanes_per_row(n);
    prof.skip();
    if (row_kernel(batch, n)) {
      hipLaunchKernelGGL((k_row<T, W, D, kRowP>), dim3((unsigned)batch), dim3(kRowMax / kRowP), 0, s, y, w, z, bstart,
                         rflags, (int)n, row_walk ? 1 : 0);
    } else {
      const int R = kWave / L;
      const int64_t tiles = (batch + R - 1) / R;
      hipLaunchKernelGGL((k_wave<T, W, D>), dim3((unsigned)tiles), dim3(kWave), 0, s, y, w, z, bstart,
                         rflags, batch, n, L);
    }
    prof.mark(1);
    return hipGetLastError() == hipSuccess ? ISO_OK : ISO_EHIP;
  }
  const int m = (int)Lay.m;
  const int nblk = (int)Lay.nblk;
  const int64_t G = batch * (int64_t)m;
  ChunkOut co;
  co.tot = (double2*)(ws + Lay.o_tot);
  co.nverts = (int*)(ws + Lay.o_nv);
  co.cflags = (uint32_t*)(ws + Lay.o_cf);
  co.desc = (Desc*)(ws + Lay.o_desc);
  co.nseg = (int*)(ws + Lay.o_nseg);
  co.lk = (uint16_t*)(ws + Lay.o_lk);
  co.lx = (double*)(ws + Lay.o_lx);
  co.ly = (double*)(ws + Lay.o_ly);
  co.mask = (uint32_t*)(ws + Lay.o_mask);
  co.mcnt = (uint16_t*)(ws + Lay.o_mcnt);
  co.lsx = (double*)(ws + Lay.o_lsx);
  co.lsy = (double*)(ws + Lay.o_lsy);
  co.ckx = (double*)(ws + Lay.o_ckx);
  co.cky = (double*)(ws + Lay.o_cky);
  co.ztile = (uint32_t*)(ws + Lay.o_zt);
  co.dform = (uint8_t*)(ws + Lay.o_df);
  co.bnd = (double4*)(ws + Lay.o_bnd);
  co.bndk = (int2*)(ws + Lay.o_bndk);
  co.G = G;
  double4* start = (double4*)(ws + Lay.o_start);
  double4* bsum = (double4*)(ws + Lay.o_bsum);
  uint32_t* bflag = (uint32_t*)(ws + Lay.o_bflag);
  EndInfo* ends = (EndInfo*)(ws + Lay.o_ends);

  hipLaunchKernelGGL((k_increasing<T, W, D>), dim3((unsigned)G), dim3(kIncWaves * kWave), 0, s, y, w, z, n,
                     m, co);
  prof.mark(1);
  hipLaunchKernelGGL((k_chunk<T, W, D, false>), dim3((unsigned)G), dim3(kWave), 0, s, y, w, z, n, m, co);
  prof.mark(1);
  hipLaunchKernelGGL((k_chunk<T, W, D, true>), dim3((unsigned)G), dim3(kWave), 0, s, y, w, z, n, m, co);
  prof.mark(1);
  if (nblk == 1) {  // rows of at most kScanBlock chunks: one launch
    hipLaunchKernelGGL(k_scan_apply<true>, dim3((unsigned)batch), dim3(kScanThreads), 0, s, co.tot, co.tot + G,
                       bsum, bflag, co.cflags, start, rflags, m, nblk);
  } else {
    hipLaunchKernelGGL(k_scan_reduce, dim3((unsigned)(nblk * batch)), dim3(kScanThreads), 0,
                       s, co.tot, co.tot + G, co.cflags, bsum, bflag, m, nblk);
    hipLaunchKernelGGL(k_scan_apply<false>, dim3((unsigned)(nblk * batch)), dim3(kScanThreads), 0, s,
                       co.tot, co.tot + G, bsum, bflag, co.cflags, start, rflags, m, nblk);
  }
  prof.mark(nblk == 1 ? 1 : 2);
  VertexStore<T, W, D> S;
  S.desc = co.desc;
  S.nseg = co.nseg;
  S.nverts = co.nverts;
  S.dense = co.dform;
  S.lx = co.lx;
  S.ly = co.ly;
  S.lk = co.lk;
  S.mask = co.mask;
  S.mcnt = co.mcnt;
  S.lsx = co.lsx;
  S.lsy = co.lsy;
  S.ckx = co.ckx;
  S.cky = co.cky;
  S.bnd = co.bnd;
  S.bndk = co.bndk;
  S.tot = co.tot;
  S.start = start;
  S.y = y;
  S.w = w;
  S.n = n;
  S.m = m;
  S.G = G;
  // the merge levels, kMergeGroup per launch (a workgroup per subtree)
  int levels = 0;
  while ((1 << levels) < m) ++levels;
  int launches = 0;
  for (int r0 = 0; r0 < levels; r0 += kMergeGroup) {
    const int nlev = std::min(kMergeGroup, levels - r0);
    const int64_t span = (int64_t)1 << (r0 + nlev);
    const int64_t per_row = (m + span - 1) / span;
    hipLaunchKernelGGL((k_merge_levels<T, W, D>), dim3((unsigned)(batch * per_row)), dim3(kMergeWaves * kWave),
                       0, s, S, r0, nlev, per_row);
    ++launches;
  }
  if (launches > 0) prof.mark(launches);
  else prof.skip();
  hipLaunchKernelGGL((k_ends<T, W, D>), dim3((unsigned)((G + 255) / 256)), dim3(256), 0, s, S, ends,
                     batch);
  prof.mark(1);
  // a chunk's fit is split over up to kFitMaxSub workgroups when there are fewer than about 2048
  // chunks, so that rows of a few chunks still occupy the chip
  const int nsub = (int)std::max<int64_t>(1, std::min<int64_t>(kFitMaxSub, 2048 / std::max<int64_t>(G, 1)));
  hipLaunchKernelGGL((k_fit<T, W, D>), dim3((unsigned)(G * nsub)), dim3(kFitThreads), 0, s, S,
                     (const EndInfo*)ends, (const uint32_t*)rflags, (const uint32_t*)co.ztile, z, bstart,
                     nsub);
  prof.mark(1);
  return hipGetLastError() == hipSuccess ? ISO_OK : ISO_EHIP;
}

template <typename T, bool D>
int dispatch_fit(const void* y, const void* w, void* z, uint8_t* bstart, uint32_t* rflags,
                 int64_t batch, int64_t n, char* ws, const Layout& Lay, hipStream_t s, bool row_walk = false) {
  if (w)
    return run_fit<T, true, D>((const T*)y, (const T*)w, (T*)z, bstart, rflags, batch, n, ws, Lay, s, row_walk);
  return run_fit<T, false, D>((const T*)y, nullptr, (T*)z, bstart, rflags, batch, n, ws, Lay, s, row_walk);
}

// ---- rows of unequal lengths (iso_ragged.h)
// Rows are bucketed by ceil(log2 length), so a bucket's padded stride L is under twice any of its
// rows' lengths (rounded up to 16 bytes so padded rows stay aligned).  Buckets run one after the
// other on the stream and share one region of the workspace.
struct RagRegion {
  size_t o_y = 0, o_w = 0, o_z = 0, o_b = 0, o_f = 0, o_keys = 0, o_ws = 0, total = 0;
  Layout fit;
};

RagRegion rag_region(int64_t c, int64_t L, size_t esz, bool weighted) {
  RagRegion R;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  const size_t e = (size_t)c * (size_t)L;
  R.o_y = take(e * esz);
  R.o_w = weighted ? take(e * esz) : 0;
  R.o_z = take(e * esz);
  R.o_b = take(e);
  R.o_f = take((size_t)c * sizeof(uint32_t));
  R.o_keys = take((size_t)c * sizeof(uint64_t));
  R.fit = make_layout(c, L);
  R.o_ws = take(R.fit.total);
  R.total = off;
  return R;
}

struct RagPlan {
  struct Bucket {
    int64_t first, c, L;
  };
  std::vector<int64_t> rows;  // the buckets' rows, bucket after bucket
  std::vector<Bucket> buckets;
  size_t o_plan = 0, o_rf = 0, o_any = 0, o_region = 0, total = 0;
};

// Validates the host offsets and plans the buckets.  Returns ISO_OK or ISO_EINVAL.
int rag_plan(const int64_t* offs, int64_t batch, int dtype, bool weighted, RagPlan& P) {
  if (batch < 0 || (dtype != ISO_F32 && dtype != ISO_F64)) return ISO_EINVAL;
  if (batch > (int64_t)INT32_MAX) return ISO_EINVAL;
  if (batch == 0) return ISO_OK;
  if (!offs || offs[0] < 0) return ISO_EINVAL;
  const size_t esz = dtype == ISO_F64 ? 8 : 4;
  const int64_t align = (int64_t)(16 / esz);
  std::vector<std::vector<int64_t>> by(64);
  for (int64_t r = 0; r < batch; ++r) {
    const int64_t len = offs[r + 1] - offs[r];
    if (len < 0 || offs[r + 1] > INT64_MAX / 16) return ISO_EINVAL;
    if (len == 0) continue;
    const int k = len == 1 ? 0 : 64 - __builtin_clzll((unsigned long long)(len - 1));
    by[k].push_back(r);
  }
  size_t region = 0;
  for (int k = 0; k < 64; ++k) {
    if (by[k].empty()) continue;
    int64_t L = 0;
    for (int64_t r : by[k]) L = std::max(L, offs[r + 1] - offs[r]);
    L = (L + align - 1) / align * align;
    const int64_t c = (int64_t)by[k].size();
    if (!shape_ok(c, L, dtype)) return ISO_EINVAL;
    const int64_t tiles = (L + kRagTile - 1) / kRagTile;
    if (c > (int64_t)INT32_MAX / tiles) return ISO_EINVAL;  // one launch block per tile
    P.buckets.push_back({(int64_t)P.rows.size(), c, L});
    P.rows.insert(P.rows.end(), by[k].begin(), by[k].end());
    region = std::max(region, rag_region(c, L, esz, weighted).total);
  }
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  P.o_plan = take(((size_t)batch + 1 + P.rows.size()) * sizeof(int64_t));  // offsets, then rows
  P.o_rf = take((size_t)batch * sizeof(uint32_t));
  P.o_any = take(sizeof(uint32_t));
  P.o_region = take(region);
  P.total = off;
  return ISO_OK;
}

template <typename T, bool D>
int run_ragged(const T* y, const T* w, T* z, uint8_t* bstart, uint32_t* rf, const RagPlan& P,
               const int64_t* offs_dev, const int64_t* rows_dev, char* ws, hipStream_t s) {
  const size_t esz = sizeof(T);
  for (const RagPlan::Bucket& b : P.buckets) {
    const RagRegion R = rag_region(b.c, b.L, esz, w != nullptr);
    char* base = ws + P.o_region;
    T* yp = (T*)(base + R.o_y);
    T* wp = w ? (T*)(base + R.o_w) : nullptr;
    T* zp = (T*)(base + R.o_z);
    uint8_t* bp = (uint8_t*)(base + R.o_b);
    uint32_t* fp = (uint32_t*)(base + R.o_f);
    uint64_t* keys = (uint64_t*)(base + R.o_keys);
    RagBucket B{offs_dev, rows_dev + b.first, b.c, b.L, (b.L + kRagTile - 1) / kRagTile};
    const unsigned grid = (unsigned)(b.c * B.tiles);
    hipLaunchKernelGGL(k_rag_init, dim3((unsigned)((b.c + kRagThreads - 1) / kRagThreads)), dim3(kRagThreads), 0,
                       s, keys, b.c, D ? 1 : 0);
    hipLaunchKernelGGL((k_rag_extreme<T, D>), dim3(grid), dim3(kRagThreads), 0, s, y, B, keys);
    if (w)
      hipLaunchKernelGGL((k_rag_pack<T, true, D>), dim3(grid), dim3(kRagThreads), 0, s, y, w, B,
                         (const uint64_t*)keys, yp, wp);
    else
      hipLaunchKernelGGL((k_rag_pack<T, false, D>), dim3(grid), dim3(kRagThreads), 0, s, y, w, B,
                         (const uint64_t*)keys, yp, wp);
    if (hipGetLastError() != hipSuccess) return ISO_EHIP;
    const int rc = dispatch_fit<T, D>(yp, wp, zp, bp, fp, b.c, b.L, base + R.o_ws, R.fit, s);
    if (rc != ISO_OK) return rc;
    hipLaunchKernelGGL((k_rag_unpack<T>), dim3(grid), dim3(kRagThreads), 0, s, (const T*)zp,
                       (const uint8_t*)bp, (const uint32_t*)fp, B, z, bstart, rf);
    if (hipGetLastError() != hipSuccess) return ISO_EHIP;
  }
  return ISO_OK;
}

// ---- soft rank (iso_softrank.h)
// Sorts every row's keys (decreasing value order) and leaves perm[r * n + k] = the flat index of
// row r's k-th largest element: a stable radix sort of the value keys with the flat indices, then,
// for more than one row, a stable radix sort of those indices by row.  With tmp == nullptr only
// sets tmp_bytes.
template <typename K>
hipError_t sr_sort(K* keys, K* keys_sorted, uint32_t* idx, uint32_t* rk, uint32_t* rk_sorted, uint32_t* perm,
                   int64_t batch, int64_t n, void* tmp, size_t& tmp_bytes, hipStream_t s) {
  const size_t N = (size_t)(batch * n);
  unsigned row_bits = 0;
  while (row_bits < 32 && (1ull << row_bits) < (unsigned long long)batch) ++row_bits;
  if (tmp == nullptr) {
    size_t a = 0, b = 0;
    hipError_t e = rocprim::radix_sort_pairs(nullptr, a, keys, keys_sorted, rocprim::counting_iterator<uint32_t>(0),
                                             idx, N, 0, 8 * sizeof(K), s);
    if (e != hipSuccess) return e;
    if (batch > 1) {
      e = rocprim::radix_sort_pairs(nullptr, b, rk, rk_sorted, idx, perm, N, 0, row_bits, s);
      if (e != hipSuccess) return e;
    }
    tmp_bytes = std::max(a, b);
    return hipSuccess;
  }
  hipError_t e = rocprim::radix_sort_pairs(tmp, tmp_bytes, keys, keys_sorted, rocprim::counting_iterator<uint32_t>(0),
                                           batch > 1 ? idx : perm, N, 0, 8 * sizeof(K), s);
  if (e != hipSuccess || batch == 1) return e;
  hipLaunchKernelGGL(k_sr_rows, dim3((unsigned)((N + kSrThreads - 1) / kSrThreads)), dim3(kSrThreads), 0, s,
                     (const uint32_t*)idx, (int64_t)N, n, rk);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return rocprim::radix_sort_pairs(tmp, tmp_bytes, rk, rk_sorted, idx, perm, N, 0, row_bits, s);
}

struct SrBuffers {
  size_t o_keys = 0, o_keys2 = 0, o_idx = 0, o_rk = 0, o_rk2 = 0, o_z = 0, o_v = 0, o_rf = 0, o_ws = 0, o_tmp = 0,
         total = 0, tmp_bytes = 0;
  Layout fit;
};

template <typename T, typename K>
int run_soft_rank(const T* x, int64_t batch, int64_t n, double eps, T* r, uint32_t* perm, uint8_t* bstart,
                  uint32_t* rflags, hipStream_t s) {
  const int64_t N = batch * n;
  SrBuffers B;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  const bool device_sort = n > kSrRowMax;  // else one workgroup per row sorts in LDS
  // fp32 values in several rows: one sort of 64-bit keys (row, value key) instead of a sort by
  // value followed by a stable sort by row
  const bool row_keys = device_sort && sizeof(K) == 4 && batch > 1;
  unsigned row_bits = 0;
  while (row_bits < 32 && (1ull << row_bits) < (unsigned long long)batch) ++row_bits;
  if (device_sort) {
    const size_t ksz = row_keys ? sizeof(uint64_t) : sizeof(K);
    B.o_keys = take(N * ksz);
    B.o_keys2 = take(N * ksz);
    if (!row_keys) {
      B.o_idx = take(N * sizeof(uint32_t));
      B.o_rk = take(N * sizeof(uint32_t));
      B.o_rk2 = take(N * sizeof(uint32_t));
    }
  }
  B.o_z = take(N * sizeof(double));
  B.o_v = take(N * sizeof(double));
  B.o_rf = take(batch * sizeof(uint32_t));
  B.fit = make_layout(batch, n);
  B.o_ws = take(B.fit.total);
  if (device_sort) {
    hipError_t e;
    if (row_keys)
      e = rocprim::radix_sort_pairs(nullptr, B.tmp_bytes, (uint64_t*)nullptr, (uint64_t*)nullptr,
                                    rocprim::counting_iterator<uint32_t>(0), (uint32_t*)nullptr, (size_t)N, 0,
                                    32 + row_bits, s);
    else
      e = sr_sort<K>(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, batch, n, nullptr, B.tmp_bytes, s);
    if (e != hipSuccess) return ISO_EHIP;
    B.o_tmp = take(B.tmp_bytes);
  }
  B.total = off;
  char* buf = nullptr;
  if (hipMallocAsync((void**)&buf, B.total, s) != hipSuccess) return ISO_ENOMEM;
  int rc = ISO_OK;
  const unsigned grid = (unsigned)((N + kSrThreads - 1) / kSrThreads);
  K* keys = (K*)(buf + B.o_keys);
  double* z = (double*)(buf + B.o_z);
  double* v = (double*)(buf + B.o_v);
  if (!device_sort) {
    // one workgroup sorts each row in LDS and writes perm and z
    hipLaunchKernelGGL((k_sr_row_sort<T, K>), dim3((unsigned)batch), dim3(kSrThreads), 0, s, x, n, eps, perm, z);
    if (hipGetLastError() != hipSuccess) rc = ISO_EHIP;
  } else if (row_keys) {
    uint64_t* k64 = (uint64_t*)(buf + B.o_keys);
    hipLaunchKernelGGL(k_sr_row_keys, dim3(grid), dim3(kSrThreads), 0, s, (const float*)x, N, n, k64);
    if (hipGetLastError() != hipSuccess ||
        rocprim::radix_sort_pairs(buf + B.o_tmp, B.tmp_bytes, k64, (uint64_t*)(buf + B.o_keys2),
                                  rocprim::counting_iterator<uint32_t>(0), perm, (size_t)N, 0, 32 + row_bits,
                                  s) != hipSuccess) {
      rc = ISO_EHIP;
    }
    if (rc == ISO_OK) {
      hipLaunchKernelGGL((k_sr_problem<T>), dim3(grid), dim3(kSrThreads), 0, s, x, (const uint32_t*)perm, N, n,
                         eps, z);
      if (hipGetLastError() != hipSuccess) rc = ISO_EHIP;
    }
  } else {
    hipLaunchKernelGGL((k_sr_keys<T, K>), dim3(grid), dim3(kSrThreads), 0, s, x, N, keys);
    if (hipGetLastError() != hipSuccess ||
        sr_sort<K>(keys, (K*)(buf + B.o_keys2), (uint32_t*)(buf + B.o_idx), (uint32_t*)(buf + B.o_rk),
                   (uint32_t*)(buf + B.o_rk2), perm, batch, n, buf + B.o_tmp, B.tmp_bytes, s) != hipSuccess) {
      rc = ISO_EHIP;
    }
    if (rc == ISO_OK) {
      hipLaunchKernelGGL((k_sr_problem<T>), dim3(grid), dim3(kSrThreads), 0, s, x, (const uint32_t*)perm, N, n,
                         eps, z);
      if (hipGetLastError() != hipSuccess) rc = ISO_EHIP;
    }
  }
  if (rc == ISO_OK)
    rc = dispatch_fit<double, true>(z, nullptr, v, bstart, rflags ? rflags : (uint32_t*)(buf + B.o_rf), batch, n,
                                    buf + B.o_ws, B.fit, s);
  if (rc == ISO_OK) {
    hipLaunchKernelGGL((k_sr_combine<T>), dim3(grid), dim3(kSrThreads), 0, s, x, (const uint32_t*)perm,
                       (const double*)v, N, eps, r);
    if (hipGetLastError() != hipSuccess) rc = ISO_EHIP;
  }
  if (hipFreeAsync(buf, s) != hipSuccess && rc == ISO_OK) rc = ISO_EHIP;
  return rc;
}

bool sr_args_ok(int64_t batch, int64_t n, int dtype, double eps) {
  if (!shape_ok(batch, n, dtype)) return false;
  if (!(eps > 0.0) || !(eps < INFINITY)) return false;
  if (batch > 0 && n > (int64_t)UINT32_MAX / batch) return false;  // flat indices are 32-bit
  return true;
}

}  // namespace

extern "C" {

int iso_prof_enable(int on) {
  g_prof_on = on != 0;
  return ISO_OK;
}

int iso_prof_read(double* ms, int64_t* launches, int64_t* calls) {
  int rc = ISO_OK;
  for (ProfCall& c : g_prof_calls) {
    if (hipEventSynchronize(c.ev[c.marks - 1]) != hipSuccess) rc = ISO_EHIP;
    for (int k = 0; k + 1 < c.marks; ++k) {
      float t = 0.0f;
      if (hipEventElapsedTime(&t, c.ev[k], c.ev[k + 1]) != hipSuccess) rc = ISO_EHIP;
      if (ms) ms[k] += (double)t;
      if (launches) launches[k] += c.launches[k];
    }
    for (int k = 0; k < c.marks; ++k)
      if (c.own[k]) (void)hipEventDestroy(c.ev[k]);
  }
  if (calls) *calls += (int64_t)g_prof_calls.size();
  g_prof_calls.clear();
  return rc;
}

int iso_prof_counters(uint64_t* out, int reset) {
  if (!out) return ISO_EINVAL;
  unsigned long long h[ISO_PROF_COUNTERS];
  if (hipDeviceSynchronize() != hipSuccess) return ISO_EHIP;
  if (hipMemcpyFromSymbol(h, HIP_SYMBOL(iso::g_branch_counts), sizeof(h)) != hipSuccess) return ISO_EHIP;
  for (int i = 0; i < ISO_PROF_COUNTERS; ++i) out[i] = (uint64_t)h[i];
  if (reset) {
    const unsigned long long zero[ISO_PROF_COUNTERS] = {};
    if (hipMemcpyToSymbol(HIP_SYMBOL(iso::g_branch_counts), zero, sizeof(zero)) != hipSuccess) return ISO_EHIP;
    if (hipDeviceSynchronize() != hipSuccess) return ISO_EHIP;
  }
  return ISO_OK;
}

const char* iso_prof_stage_name(int stage) {
  static const char* names[ISO_PROF_STAGES] = {"increasing", "chunk", "exact", "scan", "merge", "ends", "fit"};
  return (stage >= 0 && stage < ISO_PROF_STAGES) ? names[stage] : "?";
}

const char* iso_strerror(int code) {
  switch (code) {
    case ISO_OK: return "ok";
    case ISO_EINVAL: return "invalid argument";
    case ISO_EWEIGHT: return "a row holds a weight <= 0";
    case ISO_ENOMEM: return "device allocation failed";
    case ISO_EHIP: return "HIP runtime error";
    case ISO_ESCRATCH: return "the call needs more workspace than iso_fit_noalloc's fixed scratch (256 MiB)";
    default: return "unknown error code";
  }
}

size_t iso_workspace_bytes(int64_t batch, int64_t n, int dtype, int weighted) {
  (void)weighted;
  if (!shape_ok(batch, n, dtype) || batch == 0 || n == 0) return 0;
  return make_layout(batch, n).total;
}

int iso_fit_ex(const void* y, const void* w, void* z, uint8_t* block_start, uint32_t* row_flags,
               int64_t batch, int64_t n, int dtype, void* ws, size_t ws_bytes, unsigned flags,
               void* stream) {
  if (!shape_ok(batch, n, dtype)) return ISO_EINVAL;
  if (flags & ~(unsigned)(ISO_FLAG_CHECK_WEIGHTS | ISO_FLAG_DECREASING | ISO_FLAG_ROW_WALK)) return ISO_EINVAL;
  if (batch == 0 || n == 0) return ISO_OK;
  if (!y || !z) return ISO_EINVAL;
  const size_t esz = dtype == ISO_F64 ? 8 : 4;
  const size_t bytes = (size_t)batch * (size_t)n * esz;
  if (overlaps(z, bytes, y, bytes) || overlaps(z, bytes, w, bytes)) return ISO_EINVAL;
  if (overlaps(block_start, (size_t)batch * (size_t)n, z, bytes)) return ISO_EINVAL;
  const Layout Lay = make_layout(batch, n);
  const bool need_ws = long_rows(n) || (flags & ISO_FLAG_CHECK_WEIGHTS) || false;
  if (need_ws) {
    if (!ws || ws_bytes < Lay.total || ((uintptr_t)ws % kAlign) != 0) return ISO_EINVAL;
  }
  char* wsb = (char*)ws;
  uint32_t* rflags = row_flags;
  if (!rflags && need_ws) rflags = (uint32_t*)(wsb + Lay.o_rflags);
  hipStream_t s = (hipStream_t)stream;
  int rc;
  const bool rw = (flags & ISO_FLAG_ROW_WALK) != 0;
  if (flags & ISO_FLAG_DECREASING)
    rc = dtype == ISO_F64 ? dispatch_fit<double, true>(y, w, z, block_start, rflags, batch, n, wsb, Lay, s, rw)
                          : dispatch_fit<float, true>(y, w, z, block_start, rflags, batch, n, wsb, Lay, s, rw);
  else
    rc = dtype == ISO_F64 ? dispatch_fit<double, false>(y, w, z, block_start, rflags, batch, n, wsb, Lay, s, rw)
                          : dispatch_fit<float, false>(y, w, z, block_start, rflags, batch, n, wsb, Lay, s, rw);
  if (rc != ISO_OK) return rc;
  if (flags & ISO_FLAG_CHECK_WEIGHTS) {
    uint32_t* any = (uint32_t*)(wsb + Lay.o_any);
    hipLaunchKernelGGL(k_flags_any, dim3(1), dim3(256), 0, s, (const uint32_t*)rflags, batch, any);
    if (hipGetLastError() != hipSuccess) return ISO_EHIP;
    uint32_t host = 0;
    if (hipMemcpyAsync(&host, any, sizeof(uint32_t), hipMemcpyDeviceToHost, s) != hipSuccess)
      return ISO_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return ISO_EHIP;
    if (host & ISO_ROW_BAD_WEIGHT) return ISO_EWEIGHT;
  }
  return ISO_OK;
}

int iso_fit_noalloc(const void* y, const void* w, void* z, uint8_t* block_start, uint32_t* row_flags,
                    int64_t batch, int64_t n, int dtype, unsigned flags, void* stream) {
  if (!shape_ok(batch, n, dtype)) return ISO_EINVAL;
  if (flags & ~(unsigned)(ISO_FLAG_CHECK_WEIGHTS | ISO_FLAG_DECREASING)) return ISO_EINVAL;
  if (batch == 0 || n == 0) return ISO_OK;
  if (!y || !z) return ISO_EINVAL;
  const size_t need = make_layout(batch, n).total;
  if (need > (size_t)ISO_NOALLOC_SCRATCH_BYTES) return ISO_ESCRATCH;
  void* ws = nullptr;
  const int rc = scratch_address((hipStream_t)stream, &ws);
  if (rc != ISO_OK) return rc;
  return iso_fit_ex(y, w, z, block_start, row_flags, batch, n, dtype, ws, (size_t)ISO_NOALLOC_SCRATCH_BYTES, flags,
                    stream);
}

int iso_fit(const void* y, const void* w, void* z, int64_t batch, int64_t n, int dtype,
            void* stream) {
  if (!shape_ok(batch, n, dtype)) return ISO_EINVAL;
  if (batch == 0 || n == 0) return ISO_OK;
  if (!y || !z) return ISO_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  const unsigned flags = w ? (unsigned)ISO_FLAG_CHECK_WEIGHTS : 0u;
  const size_t need = make_layout(batch, n).total;
  void* ws = nullptr;
  if (hipMallocAsync(&ws, need, s) != hipSuccess) return ISO_ENOMEM;
  int rc = iso_fit_ex(y, w, z, nullptr, nullptr, batch, n, dtype, ws, need, flags, stream);
  if (hipFreeAsync(ws, s) != hipSuccess && rc == ISO_OK) rc = ISO_EHIP;
  return rc;
}

int iso_vjp(const void* g, const void* y, const void* w, const void* z,
            const uint8_t* block_start, void* gy, void* gw, int64_t batch, int64_t n, int dtype,
            void* stream) {
  if (!shape_ok(batch, n, dtype)) return ISO_EINVAL;
  if (batch == 0 || n == 0) return ISO_OK;
  if (!g || !y || !z || !block_start || !gy) return ISO_EINVAL;
  if (!w && gw) return ISO_EINVAL;
  const size_t esz = dtype == ISO_F64 ? 8 : 4;
  const size_t bytes = (size_t)batch * (size_t)n * esz;
  const void* ins[5] = {g, y, w, z, block_start};
  const size_t insz[5] = {bytes, bytes, bytes, bytes, (size_t)batch * (size_t)n};
  for (int k = 0; k < 5; ++k) {
    if (overlaps(gy, bytes, ins[k], insz[k]) || overlaps(gw, bytes, ins[k], insz[k])) return ISO_EINVAL;
  }
  if (overlaps(gy, bytes, gw, bytes)) return ISO_EINVAL;
  const int64_t ntile = (n + kVjpTile - 1) / kVjpTile;
  if (batch * ntile > (int64_t)INT32_MAX) return ISO_EINVAL;
  const int64_t T = batch * ntile;
  hipStream_t s = (hipStream_t)stream;
  if (ntile == 1) {
    // rows of at most one tile: whole rows packed kVjpTile / n to a tile, so no block crosses a
    // tile; one launch and no workspace
    const int rpt = (int)(kVjpTile / n);
    const int64_t nt = (batch + rpt - 1) / rpt;
    if (nt > (int64_t)INT32_MAX) return ISO_EINVAL;
    if (dtype == ISO_F64)
      hipLaunchKernelGGL((k_vjp_apply<double, true>), dim3((unsigned)nt), dim3(kVjpThreads), 0, s, (const double*)g,
                         (const double*)y, (const double*)w, (const double*)z, block_start,
                         (const double4*)nullptr, (double*)gy, (double*)gw, n, 1, batch, rpt);
    else
      hipLaunchKernelGGL((k_vjp_apply<float, true>), dim3((unsigned)nt), dim3(kVjpThreads), 0, s, (const float*)g,
                         (const float*)y, (const float*)w, (const float*)z, block_start,
                         (const double4*)nullptr, (float*)gy, (float*)gw, n, 1, batch, rpt);
    return hipGetLastError() == hipSuccess ? ISO_OK : ISO_EHIP;
  }
  const int64_t nblk = (ntile + kVjpBlock - 1) / kVjpBlock;
  const size_t tb = align_up((size_t)T * sizeof(VjpTile));
  const size_t cb = align_up((size_t)T * sizeof(double4));
  const size_t bb = align_up((size_t)(batch * nblk) * sizeof(double4));
  void* buf = nullptr;
  if (hipMallocAsync(&buf, tb + cb + 2 * bb, s) != hipSuccess) return ISO_ENOMEM;
  VjpTile* tiles = (VjpTile*)buf;
  double4* cc = (double4*)((char*)buf + tb);
  double4* bfw = (double4*)((char*)buf + tb + cb);
  double4* bbw = (double4*)((char*)buf + tb + cb + bb);
  auto carries = [&]() {
    hipLaunchKernelGGL(k_vjp_scan_reduce, dim3((unsigned)(nblk * batch)), dim3(kVjpScanThreads),
                       0, s, (const VjpTile*)tiles, (int)ntile, (int)nblk, bfw, bbw);
    hipLaunchKernelGGL(k_vjp_scan_apply, dim3((unsigned)(nblk * batch)), dim3(kVjpScanThreads),
                       0, s, (const VjpTile*)tiles, (int)ntile, (int)nblk, (const double4*)bfw,
                       (const double4*)bbw, cc);
  };
  if (dtype == ISO_F64) {
    hipLaunchKernelGGL((k_vjp_tiles<double>), dim3((unsigned)T), dim3(kVjpThreads), 0, s, (const double*)g,
                       (const double*)w, block_start, n, (int)ntile, tiles);
    carries();
    hipLaunchKernelGGL((k_vjp_apply<double>), dim3((unsigned)T), dim3(kVjpThreads), 0, s, (const double*)g,
                       (const double*)y, (const double*)w, (const double*)z, block_start,
                       (const double4*)cc, (double*)gy, (double*)gw, n, (int)ntile);
  } else {
    hipLaunchKernelGGL((k_vjp_tiles<float>), dim3((unsigned)T), dim3(kVjpThreads), 0, s, (const float*)g,
                       (const float*)w, block_start, n, (int)ntile, tiles);
    carries();
    hipLaunchKernelGGL((k_vjp_apply<float>), dim3((unsigned)T), dim3(kVjpThreads), 0, s, (const float*)g,
                       (const float*)y, (const float*)w, (const float*)z, block_start,
                       (const double4*)cc, (float*)gy, (float*)gw, n, (int)ntile);
  }
  int rc = hipGetLastError() == hipSuccess ? ISO_OK : ISO_EHIP;
  if (hipFreeAsync(buf, s) != hipSuccess && rc == ISO_OK) rc = ISO_EHIP;
  return rc;
}

int iso_soft_rank(const void* x, int64_t batch, int64_t n, int dtype, double eps, void* r, uint32_t* perm,
                  uint8_t* block_start, uint32_t* row_flags, void* stream) {
  if (!sr_args_ok(batch, n, dtype, eps)) return ISO_EINVAL;
  if (batch == 0 || n == 0) return ISO_OK;
  if (!x || !r || !perm) return ISO_EINVAL;
  const size_t esz = dtype == ISO_F64 ? 8 : 4;
  const size_t N = (size_t)(batch * n);
  if (overlaps(r, N * esz, x, N * esz) || overlaps(perm, N * 4, x, N * esz) || overlaps(perm, N * 4, r, N * esz))
    return ISO_EINVAL;
  if (overlaps(block_start, N, r, N * esz) || overlaps(block_start, N, perm, N * 4)) return ISO_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == ISO_F64)
    return run_soft_rank<double, uint64_t>((const double*)x, batch, n, eps, (double*)r, perm, block_start, row_flags,
                                           s);
  return run_soft_rank<float, uint32_t>((const float*)x, batch, n, eps, (float*)r, perm, block_start, row_flags, s);
}

int iso_soft_rank_vjp(const void* g, const uint32_t* perm, const uint8_t* block_start, int64_t batch, int64_t n,
                      int dtype, double eps, void* grad, void* stream) {
  if (!sr_args_ok(batch, n, dtype, eps)) return ISO_EINVAL;
  if (batch == 0 || n == 0) return ISO_OK;
  if (!g || !perm || !block_start || !grad) return ISO_EINVAL;
  const size_t esz = dtype == ISO_F64 ? 8 : 4;
  const int64_t N = batch * n;
  if (overlaps(grad, (size_t)N * esz, g, (size_t)N * esz) || overlaps(grad, (size_t)N * esz, perm, (size_t)N * 4))
    return ISO_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  double* buf = nullptr;
  if (hipMallocAsync((void**)&buf, (size_t)N * 2 * sizeof(double), s) != hipSuccess) return ISO_ENOMEM;
  double* u = buf;
  double* au = buf + N;
  const unsigned grid = (unsigned)((N + kSrThreads - 1) / kSrThreads);
  int rc = ISO_OK;
  if (dtype == ISO_F64)
    hipLaunchKernelGGL((k_sr_gather<double>), dim3(grid), dim3(kSrThreads), 0, s, (const double*)g, perm, N, u);
  else
    hipLaunchKernelGGL((k_sr_gather<float>), dim3(grid), dim3(kSrThreads), 0, s, (const float*)g, perm, N, u);
  if (hipGetLastError() != hipSuccess) rc = ISO_EHIP;
  // A u: the block averages of u over the fit's blocks (unit weights); y and z are not used
  // without weights
  if (rc == ISO_OK) rc = iso_vjp(u, u, nullptr, u, block_start, au, nullptr, batch, n, ISO_F64, stream);
  if (rc == ISO_OK) {
    if (dtype == ISO_F64)
      hipLaunchKernelGGL((k_sr_grad<double>), dim3(grid), dim3(kSrThreads), 0, s, (const double*)u,
                         (const double*)au, perm, N, eps, (double*)grad);
    else
      hipLaunchKernelGGL((k_sr_grad<float>), dim3(grid), dim3(kSrThreads), 0, s, (const double*)u,
                         (const double*)au, perm, N, eps, (float*)grad);
    if (hipGetLastError() != hipSuccess) rc = ISO_EHIP;
  }
  if (hipFreeAsync(buf, s) != hipSuccess && rc == ISO_OK) rc = ISO_EHIP;
  return rc;
}

size_t iso_ragged_workspace_bytes(const int64_t* offsets, int64_t batch, int dtype, int weighted) {
  RagPlan P;
  if (rag_plan(offsets, batch, dtype, weighted != 0, P) != ISO_OK) return 0;
  return P.total;
}

int iso_fit_ragged(const void* values, const void* weights, const int64_t* offsets, int64_t batch,
                   int dtype, void* z, uint8_t* block_start, uint32_t* row_flags, void* ws,
                   size_t ws_bytes, unsigned flags, void* stream) {
  if (flags & ~(unsigned)(ISO_FLAG_CHECK_WEIGHTS | ISO_FLAG_DECREASING)) return ISO_EINVAL;
  RagPlan P;
  const int prc = rag_plan(offsets, batch, dtype, weights != nullptr, P);
  if (prc != ISO_OK) return prc;
  if (batch == 0) return ISO_OK;
  const size_t esz = dtype == ISO_F64 ? 8 : 4;
  const size_t nel = (size_t)offsets[batch];
  if (nel > 0 && (!values || !z)) return ISO_EINVAL;
  if (overlaps(z, nel * esz, values, nel * esz) || overlaps(z, nel * esz, weights, nel * esz)) return ISO_EINVAL;
  if (overlaps(block_start, nel, z, nel * esz)) return ISO_EINVAL;
  if (!ws || ws_bytes < P.total || ((uintptr_t)ws % kAlign) != 0) return ISO_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  char* wsb = (char*)ws;
  // the plan (offsets, then the bucket rows) goes up in one copy; the call waits for it so that
  // no host memory is referenced after it returns
  std::vector<int64_t> plan((size_t)batch + 1 + P.rows.size());
  memcpy(plan.data(), offsets, ((size_t)batch + 1) * sizeof(int64_t));
  if (!P.rows.empty()) memcpy(plan.data() + batch + 1, P.rows.data(), P.rows.size() * sizeof(int64_t));
  if (hipMemcpyAsync(wsb + P.o_plan, plan.data(), plan.size() * sizeof(int64_t), hipMemcpyHostToDevice, s) !=
      hipSuccess)
    return ISO_EHIP;
  if (hipStreamSynchronize(s) != hipSuccess) return ISO_EHIP;
  const int64_t* offs_dev = (const int64_t*)(wsb + P.o_plan);
  const int64_t* rows_dev = offs_dev + batch + 1;
  uint32_t* rf = row_flags ? row_flags : (uint32_t*)(wsb + P.o_rf);
  hipLaunchKernelGGL(k_rag_clear_flags, dim3((unsigned)((batch + kRagThreads - 1) / kRagThreads)), dim3(kRagThreads),
                     0, s, rf, batch);
  if (hipGetLastError() != hipSuccess) return ISO_EHIP;
  const bool dec = (flags & ISO_FLAG_DECREASING) != 0;
  int rc;
  if (dtype == ISO_F64)
    rc = dec ? run_ragged<double, true>((const double*)values, (const double*)weights, (double*)z, block_start, rf, P,
                                        offs_dev, rows_dev, wsb, s)
             : run_ragged<double, false>((const double*)values, (const double*)weights, (double*)z, block_start, rf, P,
                                         offs_dev, rows_dev, wsb, s);
  else
    rc = dec ? run_ragged<float, true>((const float*)values, (const float*)weights, (float*)z, block_start, rf, P,
                                       offs_dev, rows_dev, wsb, s)
             : run_ragged<float, false>((const float*)values, (const float*)weights, (float*)z, block_start, rf, P,
                                        offs_dev, rows_dev, wsb, s);
  if (rc != ISO_OK) return rc;
  if (flags & ISO_FLAG_CHECK_WEIGHTS) {
    uint32_t* any = (uint32_t*)(wsb + P.o_any);
    hipLaunchKernelGGL(k_flags_any, dim3(1), dim3(256), 0, s, (const uint32_t*)rf, batch, any);
    if (hipGetLastError() != hipSuccess) return ISO_EHIP;
    uint32_t host = 0;
    if (hipMemcpyAsync(&host, any, sizeof(uint32_t), hipMemcpyDeviceToHost, s) != hipSuccess) return ISO_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return ISO_EHIP;
    if (host & ISO_ROW_BAD_WEIGHT) return ISO_EWEIGHT;
  }
  return ISO_OK;
}

}  // extern "C"
