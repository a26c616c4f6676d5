"""GPU parity of the soft rank (iso_soft_rank, iso_soft_rank_vjp) against the oracle of
oracle/softrank.py, through the C ABI.  The page's setting (Section 7.9, Table 6): standard normal
values, eps = 1 (each row pools into one block) and eps = 1/n (most elements start a block),
rows of 10^2 to 10^6, and the training-step shapes 256 x 10^3 and 4 x 10^5.

Bars: max |r - r*| / (1 + n + max |theta|) per row, the scale of the row's problem z = s - w,
<= 1e-13 for fp64 (measured at most 7.2e-15 over these cases) and <= 2.4e-7 for fp32 (four fp32
units in the last place of that scale; the fp32 outputs measured identical to the oracle's,
which rounds its fp64 result to fp32 once); the same sort permutation; the same block starts;
gradients to 1e-10 (fp64) and 1e-6 (fp32) of their largest entry.
"""
import numpy as np
import pytest

from oracle import softrank

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {np.float32: 1e-6, np.float64: 1e-10}  # gradients, relative to their largest entry
TOL_R = {np.float32: 2.4e-7, np.float64: 1e-13}  # soft ranks, relative to the row's scale


def _gpu():
    from weighted_isotonic_regression_amd import binding

    binding.load()
    return binding


def _check(x, eps, grad=True):
    b = _gpu()
    t = x.dtype.type
    xt = torch.from_numpy(x).cuda()
    r, perm, bs, rf = b.soft_rank(xt, eps, row_flags=True)
    torch.cuda.synchronize()
    ro, permo, bso = softrank.soft_rank(x.astype(np.float64), eps, dtype=t, return_context=True)
    r = r.cpu().numpy().astype(np.float64)
    # measured against the scale of the row's problem z = s - w, as the page's Appendix C states its
    # soft-rank agreement relative to the values' scale: v = fit(z) is within the fit's bar of
    # |v| <= n + max|theta|, and r = s - v carries that absolute error also to ranks near 1
    n = x.shape[-1]
    scale = 1.0 + n + np.max(np.abs(x.astype(np.float64) / eps), axis=-1, keepdims=True)
    dev = float(np.max(np.abs(r - ro) / scale))
    assert dev <= TOL_R[t], dev
    np.testing.assert_array_equal(perm.cpu().numpy().astype(np.int64) % x.shape[-1], permo)
    np.testing.assert_array_equal(bs.cpu().numpy(), bso)
    assert np.all(rf.cpu().numpy() == 0)
    if grad:
        g = np.random.default_rng(x.size).standard_normal(x.shape).astype(t)
        gx = b.soft_rank_vjp(torch.from_numpy(g).cuda(), perm, bs, eps).cpu().numpy().astype(np.float64)
        go = softrank.soft_rank_vjp(g.astype(np.float64), permo, bso, eps)
        assert np.max(np.abs(gx - go)) <= TOL[t] * max(1.0, np.max(np.abs(go))), np.max(np.abs(gx - go))
    return r


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
@pytest.mark.parametrize("shape", [(1, 1), (3, 2), (5, 17), (4, 100), (2, 2048), (2, 2049), (1, 20000), (3, 70001)])
def test_soft_rank_shapes(shape, dtype):
    x = np.random.default_rng(shape[1]).standard_normal(shape).astype(dtype)
    for eps in (1.0, 1.0 / shape[1], 1e-3, 50.0):
        _check(x, eps)


@pytest.mark.parametrize("shape", [(256, 1000), (4, 100_000), (1, 1_000_000)])
def test_soft_rank_page_shapes_fp32(shape):
    x = np.random.default_rng(7).standard_normal(shape).astype(np.float32)
    for eps in (1.0, 1.0 / shape[1]):
        _check(x, eps, grad=shape[1] <= 100_000)


def test_soft_rank_hard_and_pooled_limits():
    b = _gpu()
    x = (np.random.default_rng(3).permutation(500).astype(np.float64) * 2.0)[None, :]
    r, _, bs = b.soft_rank(torch.from_numpy(x).cuda(), 1e-3)
    np.testing.assert_array_equal(r.cpu().numpy()[0], np.argsort(np.argsort(x[0])) + 1.0)
    assert bs.cpu().numpy().all()
    x = np.random.default_rng(4).standard_normal((3, 300))
    r, _, bs = b.soft_rank(torch.from_numpy(x).cuda(), 1e7)
    theta = x / 1e7
    np.testing.assert_allclose(r.cpu().numpy(), theta - theta.mean(axis=1, keepdims=True) + 150.5, rtol=0, atol=1e-9)
    assert bs.cpu().numpy().sum() == 3


def test_soft_rank_ties_and_flags():
    b = _gpu()
    rng = np.random.default_rng(5)
    for n, t in ((3000, np.float32), (1000, np.float64), (2048, np.float32)):  # device sort, then row sorts
        x = rng.integers(0, 7, (4, n)).astype(t)  # many ties
        r = _check(x, 0.5)
        for row in range(4):
            for v in range(7):
                sel = x[row] == v
                if sel.any():
                    assert np.ptp(r[row][sel]) == 0.0  # equal values, equal soft ranks
    x = rng.standard_normal((3, 100))
    x[1, 5] = np.nan
    r, _, _, rf = b.soft_rank(torch.from_numpy(x).cuda(), 1.0, row_flags=True)
    assert list(rf.cpu().numpy()) == [0, b.ISO_ROW_NONFINITE, 0]
    r = r.cpu().numpy()
    assert np.isnan(r[1]).all() and not np.isnan(r[[0, 2]]).any()


def test_soft_rank_autograd():
    b = _gpu()
    x = torch.randn(8, 500, dtype=torch.float64, device="cuda", requires_grad=True)
    target = torch.argsort(torch.argsort(torch.randn(8, 500, dtype=torch.float64, device="cuda"))).double() + 1
    r = b.soft_rank_fn(x, 1.0 / 500)
    loss = ((r - target) ** 2).sum()
    loss.backward()
    xn = x.detach().cpu().numpy()
    ro, permo, bso = softrank.soft_rank(xn, 1.0 / 500, return_context=True)
    go = softrank.soft_rank_vjp(2 * (ro - target.cpu().numpy()), permo, bso, 1.0 / 500)
    np.testing.assert_allclose(x.grad.cpu().numpy(), go, rtol=0, atol=1e-8 * np.abs(go).max())
