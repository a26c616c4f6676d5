"""TEST INFRASTRUCTURE ONLY: exact characterisations of the isotonic fit, used to pin the oracle.

Every function here is an independent statement of what the fit is, written out in exact
rational arithmetic (``fractions.Fraction``; an fp64 or fp32 value is a dyadic rational, so
the conversion is exact).  None of them calls ``pav``.  They are slow and meant for rows of
at most a few hundred elements.

* ``maxmin``: the max-min formula for isotonic regression,
  z_i = max_{j<=i} min_{k>=i} Av(j..k), Av the weighted mean of y_j..y_k (Robertson, Wright
  and Dykstra, "Order Restricted Statistical Inference", Thm 1.4.4).
* ``lower_hull``: the greatest convex minorant of the cumulative sum diagram ("Merge Hulls
  Without Copying Vertices: GPU Isotonic Regression", Section 1 and Section 2.1): the points
  P_0 = (0, 0), P_{k+1} = P_k + (w_k, w_k y_k); the fit of element k is the slope of the hull
  edge over [X_k, X_{k+1}]; collinear middle points are not vertices, and element k starts a
  block exactly when P_k is a vertex.
* ``minmax`` and ``upper_hull``: the same two characterisations for the decreasing fit
  (z_0 >= ... >= z_{n-1}, the direction of the page's benchmarks, Section 7.2): the min-max
  formula z_i = min_{j<=i} max_{k>=i} Av(j..k) (the theorem above with the order reversed),
  and the least concave majorant of the same diagram.
* ``kkt_residual``: the optimality certificate of the page's Section 7.6 (fourth accuracy
  measure), computed from an output alone.
* ``measures``: the page's other Section 7.6 measures (step down, deviation from a reference,
  objective excess) plus the block-mean and weighted-sum invariants.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def _fr_row(y, w):
    y = [Fraction(float(v)) for v in np.asarray(y, dtype=np.float64).ravel()]
    if w is None:
        w = [Fraction(1)] * len(y)
    else:
        w = [Fraction(float(v)) for v in np.asarray(w, dtype=np.float64).ravel()]
    if len(w) != len(y):
        raise ValueError("w must have the length of y")
    if any(wi <= 0 for wi in w):
        raise ValueError("weights must be positive")
    return y, w


def csd(y, w=None):
    """Cumulative sum diagram P_0..P_n as exact (X, Y) pairs."""
    y, w = _fr_row(y, w)
    pts = [(Fraction(0), Fraction(0))]
    for yi, wi in zip(y, w):
        x0, y0 = pts[-1]
        pts.append((x0 + wi, y0 + wi * yi))
    return pts


def maxmin(y, w=None):
    """Exact fit by the max-min block-average formula.  Returns a list of Fractions."""
    y, w = _fr_row(y, w)
    n = len(y)
    W = [Fraction(0)]
    S = [Fraction(0)]
    for yi, wi in zip(y, w):
        W.append(W[-1] + wi)
        S.append(S[-1] + wi * yi)
    z = []
    # inner[j] = min_{k>=i} Av(j..k), updated as i grows: Av(j..k) for k >= i.
    # Compute directly: for each j, the suffix minimum over k of Av(j..k).
    sufmin = []
    for j in range(n):
        row = [None] * n
        best = None
        for k in range(n - 1, j - 1, -1):
            av = (S[k + 1] - S[j]) / (W[k + 1] - W[j])
            best = av if best is None or av < best else best
            row[k] = best  # min over k' >= k of Av(j..k')
        sufmin.append(row)
    for i in range(n):
        z.append(max(sufmin[j][i] for j in range(i + 1)))
    return z


def minmax(y, w=None):
    """Exact decreasing fit by the min-max block-average formula.  Returns a list of Fractions."""
    y, w = _fr_row(y, w)
    n = len(y)
    W = [Fraction(0)]
    S = [Fraction(0)]
    for yi, wi in zip(y, w):
        W.append(W[-1] + wi)
        S.append(S[-1] + wi * yi)
    # sufmax[j][k] = max over k' >= k of Av(j..k')
    sufmax = []
    for j in range(n):
        row = [None] * n
        best = None
        for k in range(n - 1, j - 1, -1):
            av = (S[k + 1] - S[j]) / (W[k + 1] - W[j])
            best = av if best is None or av > best else best
            row[k] = best
        sufmax.append(row)
    return [min(sufmax[j][i] for j in range(i + 1)) for i in range(n)]


def _cross(o, a, b):
    return (a[0] - o[0]) * (b[1] - o[1]) - (a[1] - o[1]) * (b[0] - o[0])


def lower_hull(y, w=None):
    """Canonical lower hull of the CSD by Andrew's monotone chain, popping on cross <= 0.

    Returns (vertices, z, block_start): vertex indices into P_0..P_n, the exact fit (list of
    Fractions, slope of the hull edge over each element) and the 0/1 block-start list.
    """
    pts = csd(y, w)
    hull = []
    for k, p in enumerate(pts):
        while len(hull) >= 2 and _cross(pts[hull[-2]], pts[hull[-1]], p) <= 0:
            hull.pop()
        hull.append(k)
    n = len(pts) - 1
    z = [None] * n
    starts = [0] * n
    for a, b in zip(hull[:-1], hull[1:]):
        slope = (pts[b][1] - pts[a][1]) / (pts[b][0] - pts[a][0])
        for i in range(a, b):
            z[i] = slope
        if a < n:
            starts[a] = 1
    return hull, z, starts


def upper_hull(y, w=None):
    """Canonical upper hull (least concave majorant) of the CSD, popping on cross >= 0.

    Returns (vertices, z, block_start) as ``lower_hull`` does, for the decreasing fit.
    """
    pts = csd(y, w)
    hull = []
    for k, p in enumerate(pts):
        while len(hull) >= 2 and _cross(pts[hull[-2]], pts[hull[-1]], p) >= 0:
            hull.pop()
        hull.append(k)
    n = len(pts) - 1
    z = [None] * n
    starts = [0] * n
    for a, b in zip(hull[:-1], hull[1:]):
        slope = (pts[b][1] - pts[a][1]) / (pts[b][0] - pts[a][0])
        for i in range(a, b):
            z[i] = slope
        if a < n:
            starts[a] = 1
    return hull, z, starts


def blocks_from_exact(z):
    """Block starts of an exact fit: maximal runs of equal values."""
    return [1 if i == 0 or z[i] != z[i - 1] else 0 for i in range(len(z))]


def kkt_residual(y, w, z, decreasing=False):
    """Largest violation of the optimality certificate of an output z (0 for an empty row).

    Two parts, the larger of which is returned:
      stationarity  lambda_i = -2 sum_{j<=i} w_j (z_j - y_j) must be >= 0, zero at the last
                    element and zero wherever z steps up (z_{i+1} > z_i); violations are
                    relative to 2 * sum w |y|;
      feasibility   z must be non-decreasing; the largest step down is relative to max |y|.
    Feasibility plus stationarity prove optimality of the convex problem.  For the decreasing
    fit the sign of lambda flips, the steps that free it are steps down, and feasibility asks
    for a non-increasing z.  Sums use 80-bit extended precision.
    """
    y = np.asarray(y, dtype=np.float64).ravel()
    z = np.asarray(z, dtype=np.float64).ravel()
    n = y.size
    if n == 0:
        return 0.0
    w = np.ones(n) if w is None else np.asarray(w, dtype=np.float64).ravel()
    ld = np.longdouble
    terms = w.astype(ld) * (z.astype(ld) - y.astype(ld))
    lam = -2 * np.cumsum(terms)
    if decreasing:
        lam = -lam
    scale = 2 * np.sum(w.astype(ld) * np.abs(y.astype(ld)))
    if scale == 0:
        scale = ld(1)
    viol = np.maximum(-lam, 0)
    res = max(float(viol.max()), float(abs(lam[-1])))
    up = (z[1:] < z[:-1]) if decreasing else (z[1:] > z[:-1])
    if np.any(up):
        res = max(res, float(np.abs(lam[:-1][up]).max()))
    steps = np.diff(z)
    against = float(np.max(steps if decreasing else -steps, initial=0.0))
    ymax = float(np.max(np.abs(y)))
    feas = max(against, 0.0) / (ymax if ymax > 0 else 1.0)
    return max(float(res / scale), feas)


def measures(y, w, z, z_ref=None, block_start=None, eps=None):
    """The accuracy measures of the page's Section 7.6 plus the oracle invariants.

    Returns a dict with:
      step_down   largest z_i - z_{i+1} > 0, relative to max |y|
      deviation   max_i |z_i - z_ref_i| / (1 + |z_ref_i|)   (if z_ref is given)
      objective   excess of sum w (z - y)^2 over the reference's, relative to it, or to
                  eps * sum w y^2 where that is larger (eps = unit roundoff of the type)
      kkt         kkt_residual(y, w, z)
      block_mean  largest |z_i - mean of y over i's block| / (1 + mean of |y| over the block)
                  (if block_start; the scale is the block's own magnitude, so cancellation
                  inside a block does not inflate the measure)
      sum_wz      |sum w z - sum w y| / sum w |y|
    """
    y = np.asarray(y, dtype=np.float64).ravel()
    z = np.asarray(z, dtype=np.float64).ravel()
    n = y.size
    w_ = np.ones(n) if w is None else np.asarray(w, dtype=np.float64).ravel()
    out = {}
    ymax = float(np.max(np.abs(y))) if n else 0.0
    sd = float(np.max(z[:-1] - z[1:])) if n > 1 else 0.0
    out["step_down"] = max(sd, 0.0) / (ymax if ymax > 0 else 1.0)
    if z_ref is not None:
        zr = np.asarray(z_ref, dtype=np.float64).ravel()
        out["deviation"] = float(np.max(np.abs(z - zr) / (1 + np.abs(zr)))) if n else 0.0
        ld = np.longdouble
        obj = np.sum(w_.astype(ld) * (z.astype(ld) - y.astype(ld)) ** 2)
        obj_ref = np.sum(w_.astype(ld) * (zr.astype(ld) - y.astype(ld)) ** 2)
        e = eps if eps is not None else np.finfo(np.float64).eps / 2
        denom = max(float(obj_ref), e * float(np.sum(w_.astype(ld) * y.astype(ld) ** 2)), 1e-300)
        out["objective"] = float(obj - obj_ref) / denom
    out["kkt"] = kkt_residual(y, w, z)
    if block_start is not None and n:
        bs = np.asarray(block_start).ravel().astype(bool)
        bs = bs.copy()
        bs[0] = True
        ids = np.cumsum(bs) - 1
        W = np.bincount(ids, weights=w_)
        S = np.bincount(ids, weights=w_ * y)
        A = np.bincount(ids, weights=w_ * np.abs(y))
        mean = S[ids] / W[ids]
        out["block_mean"] = float(np.max(np.abs(z - mean) / (1 + A[ids] / W[ids])))
    denom = float(np.sum(w_ * np.abs(y))) or 1.0
    out["sum_wz"] = float(abs(np.sum(w_ * z) - np.sum(w_ * y))) / denom
    return out
