"""GPU parity of the decreasing direction (ISO_FLAG_DECREASING, z_0 >= ... >= z_{n-1}, the
direction of the page's benchmarks, Section 7.2 and Table 1) against the oracle's decreasing
PAV, through the C ABI.  The bars are those of the increasing fit.  The library computes the
decreasing fit as the negated increasing fit of -y, so it is also checked to be that exact
mirror, bit for bit, including the block starts.
"""
import numpy as np
import pytest

import oracle
from tests.test_gpu_fit import _gpu, check, gpu_fit
from weighted_isotonic_regression_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SIZES = [1, 2, 33, 64, 65, 2047, 2048, 2049, 4097, 16383, 16384, 16385, 49153, 100003]


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("n", SIZES)
def test_decreasing_noise_sizes(n, dtype):
    batch = 3 if n < 100000 else 1
    for wk in ("unit", "uniform"):
        y, w = W.family("noise", batch, n, seed=n + 7, dtype=dtype, wkind=wk)
        check(y, None if wk == "unit" else w, decreasing=True)


@pytest.mark.parametrize("fam", W.FAMILIES)
@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_decreasing_families(fam, dtype):
    for n in (700, 70001):
        for wk in ("unit", "integer"):
            y, w = W.family(fam, 2, n, seed=n + 3, dtype=dtype, wkind=wk)
            cancel = fam == "cancel"
            tol = (1.4e-15 if dtype == "f64" else 1e-7) if cancel else None
            check(y, None if wk == "unit" else w, exact_partition=fam in ("integer", "constant"), tol=tol,
                  kkt=not cancel, scale_abs=cancel, decreasing=True)


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_decreasing_rows_of_whole_diagram_chunks(dtype):
    """Strictly decreasing rows: every full chunk (and the 100-element tail) is a whole-diagram
    hull of -y, every element its own block, z = y exactly with unit weights.  Then the same rows
    with one tie, drop or cliff, at chunk starts, middles and ends."""
    C = 16384
    n = 3 * C + 100
    t = np.float32 if dtype == "f32" else np.float64
    base = -np.arange(n, dtype=np.float64) / n
    y = np.stack([base, 2.0 * base]).astype(t)
    z, bs = check(y, None, exact_partition=True, decreasing=True)
    assert bs.all()
    np.testing.assert_array_equal(z, y)
    rows = []
    for pos, kind in [(C, "tie"), (C + C // 2 - 1, "rise"), (2 * C - 1, "tie"), (3 * C - 1, "rise"),
                      (C - 1, "rise"), (2 * C + 5, "cliff")]:
        r = base.copy()
        if kind == "tie":
            r[pos] = r[pos - 1]
        elif kind == "rise":
            r[pos] = r[pos - 1] + 1e-3
        else:
            r[pos] = 5.0
        rows.append(r)
    y = np.stack(rows).astype(t)
    w = np.random.default_rng(12).uniform(0.5, 2.0, size=y.shape).astype(t)
    check(y, w, decreasing=True)
    check(y, None, decreasing=True)


@pytest.mark.parametrize("n", [16, 2000, 16385, 300001])
@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_decreasing_is_the_exact_mirror(n, dtype):
    batch = 64 if n == 16 else 2
    for fam in ("sawtooth", "integer"):
        for wk in ("unit", "uniform"):
            y, w = W.family(fam, batch, n, seed=n + 1, dtype=dtype, wkind=wk)
            ww = None if wk == "unit" else w
            zd, bd, fd = gpu_fit(y, ww, decreasing=True)
            zi, bi, fi = gpu_fit(-y, ww)
            np.testing.assert_array_equal(zd, -zi)
            np.testing.assert_array_equal(bd, bi)
            np.testing.assert_array_equal(fd, fi)


def test_decreasing_unweighted_fp32_1e7():
    """The setting of the page's Table 1 comparison: one row of 10^7, decreasing, unweighted, fp32
    (synthetic noise about a falling trend)."""
    y, _ = W.family("noise", 1, 10_000_000, seed=31, dtype="f32", wkind="unit")
    y = (y - 1e-7 * np.arange(10_000_000, dtype=np.float64)).astype(np.float32)
    check(y, None, kkt=False, decreasing=True)


def test_decreasing_short_rows_65536x16():
    y, w = W.short_rows_16()
    check(y, w, decreasing=True)
    check(y, None, decreasing=True)


def test_decreasing_mixed_1e8():
    y, w = W.mixed_1e8()
    check(y, w, kkt=False, decreasing=True)


def test_decreasing_bad_rows_flagged():
    b = _gpu()
    for n in (10, 3000):
        y, w = W.family("noise", 3, n, seed=8, dtype="f64", wkind="uniform")
        y[1, n // 3] = np.inf
        w[2, 0] = 0.0
        z, bs, rf = gpu_fit(y, w, decreasing=True)
        assert list(rf) == [0, b.ISO_ROW_NONFINITE, b.ISO_ROW_BAD_WEIGHT]
        assert np.all(np.isnan(z[1])) and np.all(np.isnan(z[2])) and bs[1:].sum() == 0
        zo = oracle.pav(y[0], w[0], decreasing=True)
        assert np.max(np.abs(z[0] - zo) / (1 + np.abs(zo))) <= 1e-10


@pytest.mark.parametrize("n", [700, 40000])
def test_vjp_of_the_decreasing_fit(n):
    """iso_vjp takes no direction: with the decreasing fit's block starts it matches the oracle's
    block-averaging backward (pinned against finite differences of the decreasing fit)."""
    b = _gpu()
    y, w = W.family("noise", 3, n, seed=n, dtype="f64", wkind="uniform")
    g = np.random.default_rng(n).standard_normal(y.shape)
    yt, wt, gt = (torch.from_numpy(a).cuda() for a in (y, w, g))
    z, bs = b.fit(yt, wt, block_starts=True, decreasing=True)
    gy, gw = b.vjp(gt, yt, wt, z, bs)
    torch.cuda.synchronize()
    gyo, gwo = oracle.vjp(g, y, w, z.cpu().numpy(), bs.cpu().numpy())
    assert np.max(np.abs(gy.cpu().numpy() - gyo) / (1 + np.abs(gyo))) <= 1e-12
    assert np.max(np.abs(gw.cpu().numpy() - gwo) / (1 + np.abs(gwo))) <= 1e-12
