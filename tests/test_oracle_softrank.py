"""Pins of the soft-rank oracle (oracle/softrank.py) to facts outside itself (no GPU).

The soft rank of Section 7.9 of the page is the Euclidean projection of theta = x / eps onto the
permutahedron, the convex hull of the permutations of w = (n, ..., 1).  The pins:
  * the projection's characterisation on tiny rows: r lies in the permutahedron (its sum is
    sum(w) and its sorted partial sums are majorized by w's), and <theta - r, p - r> <= 0 for
    every vertex p (all n! permutations of w), which makes r the nearest point;
  * closed forms: tiny eps gives the hard ranks (n for the largest); huge eps pools each row into
    one block, r = theta - mean(theta) + (n + 1) / 2;
  * permutation equivariance and shift invariance in x;
  * the backward against central finite differences;
  * plausible mistakes (w ascending, the increasing fit, no unsorting) planted in copies of the
    steps fail the pins.
"""
import itertools

import numpy as np
import pytest

import oracle
from oracle import softrank


def _in_permutahedron(r, tol):
    n = r.size
    w = np.arange(n, 0, -1, dtype=np.float64)
    if abs(r.sum() - w.sum()) > tol:
        return False
    cr = np.cumsum(np.sort(r)[::-1])
    cw = np.cumsum(w)
    return bool(np.all(cr <= cw + tol))


def _is_projection(theta, r, tol=1e-9):
    n = r.size
    w = np.arange(n, 0, -1, dtype=np.float64)
    if not _in_permutahedron(r, tol):
        return False
    d = theta - r
    return all(d @ (np.array(p) - r) <= tol * (1 + np.abs(theta).max()) for p in itertools.permutations(w))


def test_projection_characterisation_on_tiny_rows():
    rng = np.random.default_rng(5)
    for n in range(1, 6):
        for _ in range(20):
            x = rng.standard_normal(n) * rng.choice([0.1, 1.0, 5.0])
            for eps in (0.05, 0.5, 1.0, 10.0):
                r = softrank.soft_rank(x, eps)
                assert _is_projection(x / eps, r), (x, eps, r)
    # ties: equal values get equal soft ranks
    x = np.array([0.3, 1.0, 0.3, -2.0, 1.0])
    r = softrank.soft_rank(x, 0.7)
    assert _is_projection(x / 0.7, r) and r[0] == r[2] and r[1] == r[4]


def test_closed_forms():
    rng = np.random.default_rng(6)
    x = rng.permutation(50).astype(np.float64) * 3.0
    r = softrank.soft_rank(x, 1e-3)
    np.testing.assert_array_equal(r, np.argsort(np.argsort(x)) + 1.0)  # hard ranks, n for the largest
    x = rng.standard_normal((3, 40))
    eps = 1e6
    r = softrank.soft_rank(x, eps)
    theta = x / eps
    expect = theta - theta.mean(axis=1, keepdims=True) + (40 + 1) / 2.0
    assert np.allclose(r, expect, rtol=0, atol=1e-12)


def test_equivariance_and_shift():
    rng = np.random.default_rng(7)
    x = rng.standard_normal(300)
    r = softrank.soft_rank(x, 0.01)
    pi = rng.permutation(300)
    np.testing.assert_allclose(softrank.soft_rank(x[pi], 0.01), r[pi], rtol=0, atol=1e-9)
    np.testing.assert_allclose(softrank.soft_rank(x + 0.25, 0.01), r, rtol=0, atol=1e-9)


def test_backward_against_finite_differences():
    rng = np.random.default_rng(8)
    for n, eps in ((6, 0.3), (25, 0.05), (40, 2.0)):
        x = rng.standard_normal(n)
        g = rng.standard_normal(n)
        r, perm, bs = softrank.soft_rank(x, eps, return_context=True)
        grad = softrank.soft_rank_vjp(g, perm, bs, eps)
        h = 1e-7
        fd = np.array([g @ (softrank.soft_rank(x + h * e, eps) - softrank.soft_rank(x - h * e, eps)) / (2 * h)
                       for e in np.eye(n)])
        assert np.allclose(grad, fd, atol=1e-5), (n, eps)


def _mutant(kind):
    def f(x, eps):
        theta = np.asarray(x, dtype=np.float64) / eps
        n = theta.size
        perm = np.argsort(-theta, kind="stable")
        s = theta[perm]
        w = np.arange(1, n + 1, dtype=np.float64) if kind == "w_ascending" else np.arange(n, 0, -1, dtype=np.float64)
        v = oracle.pav(s - w, decreasing=kind != "increasing_fit")
        if kind == "no_unsort":
            return s - v
        r = np.empty_like(theta)
        r[perm] = s - v
        return r
    return f


@pytest.mark.parametrize("kind", ["w_ascending", "increasing_fit", "no_unsort"])
def test_planted_mistakes_fail_the_pins(kind):
    f = _mutant(kind)
    rng = np.random.default_rng(9)
    failed = False
    for n in range(2, 6):
        for _ in range(10):
            x = rng.standard_normal(n)
            for eps in (0.05, 1.0):
                if not _is_projection(x / eps, f(x, eps)):
                    failed = True
    assert failed
    # the unmutated steps pass the same pins
    assert all(_is_projection(x / 1.0, softrank.soft_rank(x, 1.0)) for x in rng.standard_normal((10, 4)))
