/*
 * TEST INFRASTRUCTURE ONLY.  CPU oracle for batched weighted L2 isotonic
 * regression.  Only tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg may load or call this file; the GPU library never does.
 *
 * What it computes ("Merge Hulls Without Copying Vertices: GPU Isotonic
 * Regression", Section 1 and Section 8 "Isotonic regression"): for every row,
 *
 *     z* = argmin_z  sum_i w_i (z_i - y_i)^2   subject to z_0 <= ... <= z_{n-1},
 *
 * with w_i > 0 (w == NULL means unit weights).  The objective is strictly
 * convex, so z* is unique.  The classical sequential algorithm the page names,
 * pool adjacent violators, reaches it exactly (up to rounding): scan the row
 * once, keep a stack of blocks, and merge the top two blocks while their means
 * violate the order.
 *
 * Direction.  The page's benchmarks fit the decreasing direction (Section 7.2,
 * Table 1; the soft rank of Section 7.9 too): z_0 >= ... >= z_{n-1}.  Pool
 * adjacent violators fits it directly with the order reversed: two neighbouring
 * blocks violate it when the lower one's mean is <= the top one's.
 *
 * Canonical partition (Section 2.1 of the page: a point on the segment between
 * its neighbours is not a vertex): two neighbouring blocks with EQUAL means are
 * pooled, so adjacent blocks of the result have strictly increasing (decreasing
 * fit: strictly decreasing) means.  An
 * element starts a block exactly when its left point of the cumulative sum
 * diagram is a vertex of the canonical lower hull; element 0 always does.
 *
 * Arithmetic: plain fp64.  Block sums W = sum w, S = sum w*y are accumulated in
 * scan order, means are compared by cross-multiplication (S_p*W_t >= S_t*W_p),
 * and z = S/W is one correctly rounded division.  For integer-valued y and w
 * whose block sums and cross products stay below 2^53 every step is exact, so
 * the partition is the exact one.
 *
 * Row handling: a row holding a non-finite y or w, or a weight <= 0, gets an
 * all-NaN z, no block starts, and a flag (bit 0: non-finite value, bit 1:
 * weight <= 0).  Other rows are unaffected.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#define ORACLE_FLAG_NONFINITE 1u
#define ORACLE_FLAG_WEIGHT 2u

/* One row.  Scratch arrays hold up to n blocks.  decreasing != 0 fits the
 * decreasing direction. */
static uint32_t pav_row(const double *y, const double *w, int64_t n, double *z,
                        uint8_t *block_start, int64_t *bstart, double *bw,
                        double *bs, int decreasing) {
  uint32_t flag = 0;
  for (int64_t i = 0; i < n; ++i) {
    double wi = w ? w[i] : 1.0;
    if (!isfinite(y[i]) || !isfinite(wi)) flag |= ORACLE_FLAG_NONFINITE;
    else if (!(wi > 0.0)) flag |= ORACLE_FLAG_WEIGHT;
  }
  if (block_start)
    for (int64_t i = 0; i < n; ++i) block_start[i] = 0;
  if (flag) {
    for (int64_t i = 0; i < n; ++i) z[i] = NAN;
    return flag;
  }

  int64_t top = -1; /* index of the top block on the stack */
  for (int64_t k = 0; k < n; ++k) {
    double wk = w ? w[k] : 1.0;
    ++top;
    bstart[top] = k;
    bw[top] = wk;
    bs[top] = wk * y[k];
    /* Pool while the block below has a mean >= the top block's mean (decreasing
     * fit: <=). */
    while (top >= 1 && (decreasing ? bs[top - 1] * bw[top] <= bs[top] * bw[top - 1]
                                   : bs[top - 1] * bw[top] >= bs[top] * bw[top - 1])) {
      bw[top - 1] += bw[top];
      bs[top - 1] += bs[top];
      --top;
    }
  }

  for (int64_t b = 0; b <= top; ++b) {
    int64_t lo = bstart[b];
    int64_t hi = (b < top) ? bstart[b + 1] : n;
    double mean = bs[b] / bw[b];
    for (int64_t i = lo; i < hi; ++i) z[i] = mean;
    if (block_start) block_start[lo] = 1;
  }
  return flag;
}

/*
 * iso_oracle_fit_dir: rows of common length n, row-major [batch, n], fp64.
 *   y          input values (required)
 *   w          weights, or NULL for unit weights
 *   z          output fit (required, may not alias y or w)
 *   block_start  output, 1 byte per element, or NULL
 *   row_flags  output, one uint32 per row, or NULL
 *   decreasing 0: non-decreasing fit; otherwise non-increasing
 * Returns 0 on success, -1 if scratch could not be allocated, -2 on bad sizes.
 */
int iso_oracle_fit_dir(const double *y, const double *w, double *z,
                       uint8_t *block_start, uint32_t *row_flags, int64_t batch,
                       int64_t n, int decreasing) {
  if (batch < 0 || n < 0) return -2;
  if (batch == 0 || n == 0) return 0;
  int64_t *bstart = (int64_t *)malloc((size_t)n * sizeof(int64_t));
  double *bw = (double *)malloc((size_t)n * sizeof(double));
  double *bs = (double *)malloc((size_t)n * sizeof(double));
  if (!bstart || !bw || !bs) {
    free(bstart);
    free(bw);
    free(bs);
    return -1;
  }
  for (int64_t r = 0; r < batch; ++r) {
    const double *yr = y + r * n;
    const double *wr = w ? w + r * n : NULL;
    uint32_t f = pav_row(yr, wr, n, z + r * n,
                         block_start ? block_start + r * n : NULL, bstart, bw,
                         bs, decreasing);
    if (row_flags) row_flags[r] = f;
  }
  free(bstart);
  free(bw);
  free(bs);
  return 0;
}

/* iso_oracle_fit: the non-decreasing fit (iso_oracle_fit_dir with decreasing = 0). */
int iso_oracle_fit(const double *y, const double *w, double *z,
                   uint8_t *block_start, uint32_t *row_flags, int64_t batch,
                   int64_t n) {
  return iso_oracle_fit_dir(y, w, z, block_start, row_flags, batch, n, 0);
}

/*
 * iso_oracle_vjp: the backward of the fit ("Merge Hulls Without Copying
 * Vertices", Section 6 "Gradient").  The fit is constant on blocks, each block
 * the weighted mean of y over it, so its Jacobian averages over blocks.  With
 * G and W the sums of g and w over the block holding element i:
 *     gy_i = w_i * G / W,      gw_i = (y_i - z_i) * G / W.
 * Blocks are read from block_start (1 where a block starts).  w == NULL means
 * unit weights (then W is the block length and gw must be NULL).
 */
int iso_oracle_vjp(const double *g, const double *y, const double *w,
                   const double *z, const uint8_t *block_start, double *gy,
                   double *gw, int64_t batch, int64_t n) {
  if (batch < 0 || n < 0) return -2;
  for (int64_t r = 0; r < batch; ++r) {
    const double *gr = g + r * n;
    const uint8_t *br = block_start + r * n;
    int64_t lo = 0;
    while (lo < n) {
      int64_t hi = lo + 1;
      while (hi < n && !br[hi]) ++hi;
      double G = 0.0, W = 0.0;
      for (int64_t i = lo; i < hi; ++i) {
        G += gr[i];
        W += w ? w[r * n + i] : 1.0;
      }
      for (int64_t i = lo; i < hi; ++i) {
        double wi = w ? w[r * n + i] : 1.0;
        if (gy) gy[r * n + i] = wi * G / W;
        if (gw) gw[r * n + i] = (y[r * n + i] - z[r * n + i]) * G / W;
      }
      lo = hi;
    }
  }
  return 0;
}
