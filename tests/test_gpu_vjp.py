"""GPU parity of the backward (iso_vjp) against the oracle's block averaging over the same
block starts ("Merge Hulls Without Copying Vertices", Section 6 "Gradient"; its Appendix C
validates with block sums over the GPU's own block starts on every family)."""
import numpy as np
import pytest

import oracle
from weighted_isotonic_regression_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _b():
    from weighted_isotonic_regression_amd import binding

    binding.load()
    return binding


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("n", [1, 7, 33, 2048, 2049, 5000, 70001])
@pytest.mark.parametrize("fam", ["noise", "sawtooth", "constant", "increasing", "integer"])
def test_vjp_matches_block_averaging(fam, n, dtype):
    b = _b()
    batch = 3
    rng = np.random.default_rng(n)
    for wk in ("unit", "uniform"):
        y, w = W.family(fam, batch, n, seed=n + 2, dtype=dtype, wkind=wk)
        w_ = None if wk == "unit" else w
        g = rng.standard_normal((batch, n)).astype(y.dtype)
        yt = torch.from_numpy(y).cuda()
        wt = None if w_ is None else torch.from_numpy(w_).cuda()
        gt = torch.from_numpy(g).cuda()
        z, bs = b.fit(yt, wt, block_starts=True)
        gy, gw = b.vjp(gt, yt, wt, z, bs)
        torch.cuda.synchronize()
        bs_h = bs.cpu().numpy()
        ry, rw = oracle.vjp(g.astype(np.float64), y.astype(np.float64),
                            None if w_ is None else w_.astype(np.float64), z.cpu().numpy().astype(np.float64), bs_h)
        tol = 1e-12 if dtype == "f64" else 2e-6
        gy_h = gy.cpu().numpy().astype(np.float64)
        assert np.max(np.abs(gy_h - ry) / (1 + np.abs(ry))) <= tol
        if w_ is None:
            assert gw is None
        else:
            gw_h = gw.cpu().numpy().astype(np.float64)
            assert np.max(np.abs(gw_h - rw) / (1 + np.abs(rw))) <= tol


def _check_vjp(b, y, w_, g, tol):
    yt = torch.from_numpy(y).cuda()
    wt = None if w_ is None else torch.from_numpy(w_).cuda()
    gt = torch.from_numpy(g).cuda()
    z, bs = b.fit(yt, wt, block_starts=True)
    gy, gw = b.vjp(gt, yt, wt, z, bs)
    torch.cuda.synchronize()
    ry, rw = oracle.vjp(g.astype(np.float64), y.astype(np.float64),
                        None if w_ is None else w_.astype(np.float64), z.cpu().numpy().astype(np.float64),
                        bs.cpu().numpy())
    assert np.max(np.abs(gy.cpu().numpy().astype(np.float64) - ry) / (1 + np.abs(ry))) <= tol
    if w_ is not None:
        assert np.max(np.abs(gw.cpu().numpy().astype(np.float64) - rw) / (1 + np.abs(rw))) <= tol


@pytest.mark.parametrize("fam", ["noise", "decreasing", "sawtooth"])
def test_vjp_rows_of_many_tiles(fam):
    """Rows of 3073 tiles of 2048: the carries of blocks cross the scan's blocks of 1024 tiles (the
    decreasing row is one block end to end)."""
    b = _b()
    n = 3 * 2**21 + 5
    y, w = W.family(fam, 2, n, seed=5, dtype="f64", wkind="uniform")
    g = np.random.default_rng(6).standard_normal((2, n))
    _check_vjp(b, y, w, g, 1e-12)


def test_vjp_65537_rows():
    b = _b()
    y, w = W.family("noise", 65537, 16, seed=7, dtype="f32", wkind="uniform")
    g = np.random.default_rng(8).standard_normal((65537, 16)).astype(np.float32)
    _check_vjp(b, y, w, g, 2e-6)
