"""TEST INFRASTRUCTURE ONLY: CPU oracle of the soft rank.  Only tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg may use it; the GPU library never does.

What it computes ("Merge Hulls Without Copying Vertices: GPU Isotonic Regression", Section 7.9,
the soft rank of Blondel et al. with L2 regularization of strength eps): per row, theta = x / eps
is projected onto the permutahedron of w = (n, ..., 1).  The steps, in the page's order:
  1. sort theta in decreasing order into s (a stable sort: equal values keep their order);
  2. fit the decreasing isotonic regression v of z = s - w, unit weights (the pool-adjacent-
     violators oracle, iso_oracle.c);
  3. return s - v in the original order.
``dtype`` is the precision of the problem: z is rounded to it before the fit (the page checks
its solvers against an fp64 solution of the same fp32 problem z, Appendix C), the fit and s - v
are fp64, and r is rounded to it once.

The backward: r = s - v(s - w) with s a permutation of theta, and v's Jacobian averages over the
fit's blocks (Section 6, Gradient, unit weights), so with u the cotangent in sorted order the
cotangent of x is (u - A u) / eps in the original order.
"""
from __future__ import annotations

import numpy as np

from . import native


def _rows(a):
    a = np.asarray(a, dtype=np.float64)
    return a[None, :] if a.ndim == 1 else a


def soft_rank(x, eps, *, dtype=np.float64, return_context=False):
    """Soft ranks of every row of x (1-D or [batch, n]).  Returns r (fp64 values of the given dtype,
    x's shape), and with return_context=True also (perm, block_start): perm[i, k] is the column of
    row i's k-th largest element and block_start the fit's block starts in sorted order."""
    x_in = np.asarray(x)
    x2 = _rows(x_in)
    batch, n = x2.shape
    theta = x2 / eps
    perm = np.argsort(-theta, axis=1, kind="stable")
    s = np.take_along_axis(theta, perm, axis=1)
    w = np.arange(n, 0, -1, dtype=np.float64)
    z = (s - w).astype(dtype).astype(np.float64)
    v, bs, _ = native.pav(z, None, return_blocks=True, decreasing=True)
    v = v.reshape(batch, n)
    r = np.empty_like(theta)
    np.put_along_axis(r, perm, (s - v).astype(dtype).astype(np.float64), axis=1)
    r = r.reshape(x_in.shape)
    if return_context:
        return r, perm, bs.reshape(batch, n)
    return r


def soft_rank_vjp(g, perm, block_start, eps):
    """Cotangent of x for the cotangent g of soft_rank's r (both [batch, n] or 1-D)."""
    g_in = np.asarray(g)
    g2 = _rows(g_in)
    perm = np.asarray(perm).reshape(g2.shape)
    bs = np.asarray(block_start).reshape(g2.shape)
    u = np.take_along_axis(g2, perm, axis=1)
    au, _ = native.vjp(u, u, None, u, bs)
    grad = np.empty_like(g2)
    np.put_along_axis(grad, perm, (u - au.reshape(g2.shape)) / eps, axis=1)
    return grad.reshape(g_in.shape)
