/*
 * iso.h -- C ABI of the MI355X (gfx950) batched weighted L2 isotonic regression library
 * (libiso_mi355x.so).
 *
 * The fit.  For every row of a row-major [batch, n] array,
 *
 *     z* = argmin_z  sum_i w_i (z_i - y_i)^2   subject to  z_0 <= z_1 <= ... <= z_{n-1},
 *
 * with w_i > 0 ("Merge Hulls Without Copying Vertices: GPU Isotonic Regression", Section 1).
 * z* is the slope sequence of the lower convex hull of the cumulative sum diagram
 * P_0 = (0, 0), P_{k+1} = P_k + (w_k, w_k y_k) (same page, Section 1 and Section 2.1; the
 * page's equations for the diagram were lost in extraction, this is the classical reading).
 * Element k starts a block exactly when P_k is a vertex of the canonical hull, in which a point
 * lying on the segment between its neighbours is not a vertex (Section 2.1), so neighbouring
 * blocks have strictly increasing means.
 *
 * Conventions common to every entry point
 *   - Arrays are device memory owned by the caller, contiguous, row-major [batch, n]: element
 *     (r, i) is at index r * n + i.  Indices and sizes are 64-bit.
 *   - dtype is ISO_F32 or ISO_F64 and applies to y, w, z, g, gy and gw alike.  Whatever the
 *     dtype, the diagram is accumulated in fp64 (an fp32 product w*y is exact in fp64) and every
 *     output value is one fp64 slope rounded once to dtype (round to nearest even).
 *   - stream is a hipStream_t cast to void* (NULL: the null stream).  Work is enqueued on it and
 *     the call returns without waiting, except where a synchronous check is requested.  The
 *     library keeps no pointer beyond the stream's completion of the call's work.
 *   - Errors in the arguments are returned synchronously, before anything is enqueued.
 *   - Input rows with a non-finite y or w, or a w <= 0, are flagged per row (bit 0: non-finite
 *     value, bit 1: weight <= 0) and get an all-NaN z and no block starts; other rows are fitted
 *     normally (the page's Section 6 keeps per-row NaN flags and checks weight positivity).
 *   - batch == 0 or n == 0 returns ISO_OK and enqueues nothing.
 */
#ifndef ISO_MI355X_H
#define ISO_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
enum { ISO_F32 = 0, ISO_F64 = 1 };

/* Return codes. */
enum {
  ISO_OK = 0,
  ISO_EINVAL = 1,  /* bad argument: NULL pointer, negative size, overflow, bad dtype, overlap,
                      workspace too small */
  ISO_EWEIGHT = 2, /* synchronous weight check found a row with a weight <= 0 (or non-finite) */
  ISO_ENOMEM = 3,  /* device allocation of the workspace failed (iso_fit only) */
  ISO_EHIP = 4,    /* a HIP runtime call or kernel launch failed */
  ISO_ESCRATCH = 5 /* iso_fit_noalloc: the call needs more than ISO_NOALLOC_SCRATCH_BYTES */
};

/* Bytes of the fixed device scratch of iso_fit_noalloc (256 MiB per GPU). */
enum { ISO_NOALLOC_SCRATCH_BYTES = 268435456 };

/* Flags of iso_fit_ex. */
enum {
  /* After the fit, wait for the stream and return ISO_EWEIGHT if any row holds a weight <= 0
     or a non-finite weight (the page's Section 6: weighted calls check positivity, which waits
     for the GPU). */
  ISO_FLAG_CHECK_WEIGHTS = 1u,
  /* Fit the decreasing direction instead: z_0 >= z_1 >= ... >= z_{n-1} (the page's benchmarks
     fit this direction, Section 7.2 and Table 1, as does the soft rank of Section 7.9).  It is
     computed as the negation of the increasing fit of -y; negation is exact and rounding to
     nearest is symmetric, so the result is exactly that mirror.  Block starts mark where a block
     of the decreasing fit starts; neighbouring blocks then have strictly decreasing means.
     iso_vjp needs no flag: given the block starts, its formula holds in either direction. */
  ISO_FLAG_DECREASING = 2u,
  /* For testing.  Rows of at most 4096 elements fitted one per workgroup (rows of 2049 to 4096,
     and shorter rows in batches of at most 256) find every bridge that is not a plain
     concatenation by the walk from the shared point (the page's Lemma 4.2) instead of the
     parallel search.  Where the turns are exact both give the same hull; the walk otherwise runs
     only when rounding of a near-degenerate turn leaves the parallel search inconclusive, and
     this flag lets a test check it.  No effect on other rows. */
  ISO_FLAG_ROW_WALK = 4u
};

/* Per-row flag bits written to row_flags. */
enum { ISO_ROW_NONFINITE = 1u, ISO_ROW_BAD_WEIGHT = 2u };

/*
 * iso_fit -- fit every row; the simple entry point.
 *   y      [batch, n] input values (required).
 *   w      [batch, n] weights, or NULL for unit weights.
 *   z      [batch, n] output fit (required; must not overlap y or w).
 * Scratch memory is taken from the stream-ordered allocator (hipMallocAsync/hipFreeAsync).
 * When w != NULL the call behaves as iso_fit_ex with ISO_FLAG_CHECK_WEIGHTS (it waits for the
 * stream).  Returns ISO_OK, ISO_EINVAL, ISO_EWEIGHT, ISO_ENOMEM or ISO_EHIP.
 */
int iso_fit(const void* y, const void* w, void* z, int64_t batch, int64_t n, int dtype,
            void* stream);

/*
 * iso_workspace_bytes -- size in bytes of the workspace iso_fit_ex needs for this shape
 * (weighted != 0 when w will be passed).  0 means no workspace is needed.  Returns 0 for
 * invalid shapes as well; iso_fit_ex reports those.
 */
size_t iso_workspace_bytes(int64_t batch, int64_t n, int dtype, int weighted);

/*
 * iso_fit_ex -- fit with caller-provided workspace and optional outputs.
 *   block_start  [batch, n] bytes, or NULL: 1 where an element starts a block (its left point of
 *                the diagram is a vertex of the canonical hull), else 0.  Element 0 of every
 *                valid row is 1.  Needed by iso_vjp.
 *   row_flags    [batch] uint32, or NULL: the per-row flag bits above.
 *   ws, ws_bytes device workspace of at least iso_workspace_bytes(batch, n, dtype, w != NULL)
 *                bytes, 256-byte aligned; may be NULL when that size is 0.  Its contents on entry
 *                do not matter and on return are unspecified.  Calls that share a workspace must
 *                be ordered on one stream.
 *   flags        0, or ISO_FLAG_CHECK_WEIGHTS, ISO_FLAG_DECREASING and/or ISO_FLAG_ROW_WALK.
 * Returns ISO_OK, ISO_EINVAL, ISO_EWEIGHT (only with ISO_FLAG_CHECK_WEIGHTS) or ISO_EHIP.
 */
int iso_fit_ex(const void* y, const void* w, void* z, uint8_t* block_start, uint32_t* row_flags,
               int64_t batch, int64_t n, int dtype, void* ws, size_t ws_bytes, unsigned flags,
               void* stream);

/*
 * iso_fit_noalloc -- iso_fit_ex for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels, with
 * the workspace taken from a fixed scratch array of ISO_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends.  The call itself allocates nothing.
 *   Arguments as in iso_fit_ex, without ws and ws_bytes.  The stream's device must be the
 *   current device (its scratch is looked up once per device, on the first call there).
 *   A shape whose iso_workspace_bytes exceeds ISO_NOALLOC_SCRATCH_BYTES returns ISO_ESCRATCH
 *   before anything is launched (one row of up to about 1.43e8 elements fits, and so do 1024
 *   rows of 131072).
 *   Every call on a GPU shares that GPU's scratch: calls that may overlap in time (different
 *   streams, or different host threads) race and must not be issued; calls ordered on one
 *   stream are safe.  No result depends on the scratch's previous contents.
 * Returns ISO_OK, ISO_EINVAL, ISO_ESCRATCH, ISO_EWEIGHT (only with ISO_FLAG_CHECK_WEIGHTS, which
 * waits for the stream) or ISO_EHIP.
 */
int iso_fit_noalloc(const void* y, const void* w, void* z, uint8_t* block_start, uint32_t* row_flags,
                    int64_t batch, int64_t n, int dtype, unsigned flags, void* stream);

/*
 * iso_vjp -- backward of the fit: the vector-Jacobian product with a cotangent g.  The fit is
 * constant on blocks, each the weighted mean of y over the block, so with G and W the sums of g
 * and w over the block holding element i ("Merge Hulls Without Copying Vertices", Section 6,
 * Gradient):
 *     gy_i = w_i * G / W,       gw_i = (y_i - z_i) * G / W.
 *   g, y, z      [batch, n] (z the fit of y)
 *   w            weights or NULL (unit; then W is the block's length and gw must be NULL)
 *   block_start  [batch, n] block starts written by iso_fit_ex for this y, w (required; blocks
 *                are not re-derived from z, since distinct means can round to equal values)
 *   gy           [batch, n] output (required)
 *   gw           [batch, n] output or NULL
 * Sums are taken in fp64 without atomics.  Rows of at most 2048 elements take one kernel launch
 * and no workspace; longer rows take four launches and a stream-ordered workspace allocation.
 * Returns ISO_OK, ISO_EINVAL, ISO_ENOMEM or ISO_EHIP.
 */
int iso_vjp(const void* g, const void* y, const void* w, const void* z,
            const uint8_t* block_start, void* gy, void* gw, int64_t batch, int64_t n, int dtype,
            void* stream);

/*
 * iso_fit_ragged -- fit rows of unequal lengths laid end to end ("Merge Hulls Without Copying
 * Vertices", Section 9, Limitations: the operator takes a rectangular batch, and rows of unequal
 * length are padded).  Row r is the elements offsets[r] .. offsets[r+1]-1 of the packed arrays.
 *   values       packed input values, at least offsets[batch] elements (device)
 *   weights      packed weights of the same layout, or NULL for unit weights (device)
 *   offsets      batch + 1 non-decreasing int64 offsets, offsets[0] >= 0, in HOST memory; read
 *                during the call only
 *   z            packed output fit, same layout (device; must not overlap values or weights)
 *   block_start  packed block starts, or NULL (device); as in iso_fit_ex, within each row
 *   row_flags    [batch] uint32 per-row flags, or NULL (device); an empty row gets 0
 *   ws, ws_bytes device workspace of at least iso_ragged_workspace_bytes(offsets, batch, dtype,
 *                weights != NULL) bytes, 256-byte aligned
 *   flags        0, or ISO_FLAG_CHECK_WEIGHTS and/or ISO_FLAG_DECREASING
 * Each row's fit equals its fit as a row of its own, to rounding.  Method: rows are grouped in
 * buckets of lengths within a factor of two; each bucket is copied into a rectangular buffer
 * whose rows are padded after their last element, at unit weight, with a value beyond the row's
 * range (its maximum M plus |M|/1024 + 1; for the decreasing fit its minimum minus that).  Those
 * pads never pool with the row's elements.  The bucket is fitted as by iso_fit_ex and each row's
 * part copied back.  A row whose extreme is so large that the pad overflows the element type is
 * flagged ISO_ROW_NONFINITE.  The call uploads the bucket plan and waits for the stream once
 * before enqueueing its kernels; it returns without waiting for them unless
 * ISO_FLAG_CHECK_WEIGHTS is given.  Returns ISO_OK, ISO_EINVAL (bad offsets, sizes, flags,
 * pointers or workspace), ISO_EWEIGHT or ISO_EHIP.
 */
int iso_fit_ragged(const void* values, const void* weights, const int64_t* offsets, int64_t batch,
                   int dtype, void* z, uint8_t* block_start, uint32_t* row_flags, void* ws,
                   size_t ws_bytes, unsigned flags, void* stream);

/*
 * iso_ragged_workspace_bytes -- size in bytes of the workspace iso_fit_ragged needs for these
 * host offsets (weighted != 0 when weights will be passed); 0 for invalid offsets or sizes, or
 * when batch == 0.
 */
size_t iso_ragged_workspace_bytes(const int64_t* offsets, int64_t batch, int dtype, int weighted);

/*
 * iso_soft_rank -- the soft rank with L2 regularization of every row ("Merge Hulls Without Copying
 * Vertices", Section 7.9, after Blondel et al.): the projection of theta = x / eps onto the
 * permutahedron of w = (n, ..., 1).  Per row, theta is sorted in decreasing order into s, the
 * decreasing isotonic regression v of z = s - w (unit weights) is fitted, and r = s - v is
 * returned in the original order.  z is rounded to the input type, the fit runs in fp64, and each
 * r is rounded once.  Small eps gives the hard ranks (n for the largest element); large eps pools
 * each row into one block.
 *   x            [batch, n] values (device)
 *   eps          regularization strength, finite and > 0
 *   r            [batch, n] output soft ranks (device; must not overlap x)
 *   perm         [batch, n] uint32 output (device): perm[i * n + k] is the flat index of row i's
 *                k-th largest element (ties keep their order).  Needed by iso_soft_rank_vjp.
 *   block_start  [batch, n] bytes or NULL (device): the fit's block starts, in sorted order.
 *                Needed by iso_soft_rank_vjp.
 *   row_flags    [batch] uint32 or NULL (device): ISO_ROW_NONFINITE for a row holding a non-finite
 *                value (its r is all NaN)
 * batch * n must be below 2^32.  Scratch memory (about 40 bytes per element) comes from the
 * stream-ordered allocator.  Returns ISO_OK, ISO_EINVAL, ISO_ENOMEM or ISO_EHIP.
 */
int iso_soft_rank(const void* x, int64_t batch, int64_t n, int dtype, double eps, void* r,
                  uint32_t* perm, uint8_t* block_start, uint32_t* row_flags, void* stream);

/*
 * iso_soft_rank_vjp -- backward of iso_soft_rank: with g the cotangent of r, writes the cotangent
 * of x, grad = (u - A u) / eps in the original order, where u is g in sorted order and A averages
 * over the fit's blocks (Section 6, Gradient, with unit weights).
 *   g, grad      [batch, n] (device; grad must not overlap g or perm)
 *   perm, block_start  as written by the iso_soft_rank call of the same x and eps
 * Scratch memory (16 bytes per element and the backward's own) comes from the stream-ordered
 * allocator.  Returns ISO_OK, ISO_EINVAL, ISO_ENOMEM or ISO_EHIP.
 */
int iso_soft_rank_vjp(const void* g, const uint32_t* perm, const uint8_t* block_start, int64_t batch,
                      int64_t n, int dtype, double eps, void* grad, void* stream);

/* iso_strerror -- static description of a return code. */
const char* iso_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* ISO_MI355X_H */
