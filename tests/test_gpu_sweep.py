"""GPU parity sweep: seeded random shapes over every path of the fit against the oracle, through
the C ABI.

Each case draws a row length from one of the size classes the library treats differently (1..16
four lanes per row; 17..2048 one row per workgroup of 1024 threads in batches of at most 256,
packed rows in larger ones; 2049..4096 one row per workgroup; longer rows split into chunks of
16384, with ragged tails), a batch, a family, a weight kind, a
direction and a dtype, and checks z, block starts (on integer-valued families) and row flags
against the oracle with the bars of the other parity tests.  A ragged batch mixing the classes is
checked the same way, row by row.

Weights spanning eight orders of magnitude (LogUniform[1e-4, 1e4]) are one of the four weight
kinds; every case is held to the same bars, and fp64 cases also to no step against the fitted
direction beyond a few units in the last place.
"""
import numpy as np
import pytest

import oracle
from tests.test_gpu_fit import TOL, gpu_fit
from weighted_isotonic_regression_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CLASSES = [(1, 16), (17, 2048), (2049, 4096), (4097, 8192), (8193, 70000)]
EXACT = ("integer", "constant")


def _case(rng):
    lo, hi = CLASSES[rng.integers(len(CLASSES))]
    n = int(rng.integers(lo, hi + 1))
    batch = int(rng.integers(1, max(2, min(300, 400000 // n))))
    fam = W.FAMILIES[rng.integers(len(W.FAMILIES))]
    wkind = ["unit", "uniform", "extreme", "integer"][rng.integers(4)]
    if fam == "integer":
        wkind = "integer"
    dtype = ["f32", "f64"][rng.integers(2)]
    dec = bool(rng.integers(2))
    null_w = wkind == "unit" and bool(rng.integers(2))
    return n, batch, fam, wkind, dtype, dec, null_w


def _run_case(rng, n, batch, fam, wkind, dtype, dec, null_w):
    y, w = W.family(fam, batch, n, seed=int(rng.integers(1 << 30)), dtype=dtype, wkind=wkind)
    ww = None if null_w else w
    z, bs, rf = gpu_fit(y, ww, decreasing=dec)
    zo, bo, fo = oracle.pav(y.astype(np.float64), None if ww is None else ww.astype(np.float64),
                            return_blocks=True, decreasing=dec)
    zo = zo.reshape(y.shape)
    bo = bo.reshape(y.shape)
    tag = (n, batch, fam, wkind, dtype, dec, null_w)
    np.testing.assert_array_equal(rf.astype(np.uint32), fo, err_msg=str(tag))
    zz = z.astype(np.float64)
    if fam == "cancel":  # measured against max |y| (the page's Section 7.6 measure)
        dev = float(np.max(np.abs(zz - zo)) / np.max(np.abs(y.astype(np.float64))))
        assert dev <= (1.4e-15 if dtype == "f64" else 1e-7), (tag, dev)
    else:
        dev = float(np.max(np.abs(zz - zo) / (1 + np.abs(zo))))
        assert dev <= TOL[y.dtype.type], (tag, dev)
    if dtype == "f64":
        steps = np.diff(zz, axis=1)
        wrong = float(np.max(steps if dec else -steps, initial=0.0)) / max(1.0, float(np.max(np.abs(zz))))
        assert wrong <= 1e-15, (tag, wrong)
    if fam in EXACT and wkind in ("unit", "integer"):
        np.testing.assert_array_equal(bs, bo, err_msg=str(tag))


@pytest.mark.parametrize("seed", range(12))
def test_sweep(seed):
    rng = np.random.default_rng(1000 + seed)
    for _ in range(6):
        _run_case(rng, *_case(rng))


@pytest.mark.parametrize("seed", range(6))
def test_sweep_long_row_batches(seed):
    """Batches of 1 to 4 rows of 2 to 75 chunks of 16384 with a ragged last chunk: merge trees of
    1 to 7 levels, cut into launches of three levels with one workgroup per subtree of eight
    chunks, so that a batch holds many subtrees and rows end inside a subtree."""
    rng = np.random.default_rng(3000 + seed)
    for _ in range(3):
        n = int(rng.integers(16385, 75 * 16384 + 1))
        batch = int(rng.integers(1, 5))
        _, _, fam, wkind, dtype, dec, null_w = _case(rng)
        _run_case(rng, n, batch, fam, wkind, dtype, dec, null_w)


@pytest.mark.parametrize("seed", range(4))
def test_sweep_ragged(seed):
    from weighted_isotonic_regression_amd import binding

    rng = np.random.default_rng(2000 + seed)
    lens = []
    for _ in range(40):
        lo, hi = CLASSES[rng.integers(len(CLASSES))]
        lens.append(0 if rng.integers(8) == 0 else int(rng.integers(lo, min(hi, 30000) + 1)))
    dtype = ["f32", "f64"][seed % 2]
    dec = bool(seed // 2)
    t = np.float32 if dtype == "f32" else np.float64
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    y = rng.standard_normal(int(offs[-1])).astype(t)
    w = rng.uniform(0.5, 2.0, int(offs[-1])).astype(t)
    z = binding.fit_ragged(torch.from_numpy(y).cuda(), offs, torch.from_numpy(w).cuda(), decreasing=dec)
    z = z.cpu().numpy().astype(np.float64)
    for r in range(len(lens)):
        a, e = offs[r], offs[r + 1]
        if a < e:
            zo = oracle.pav(y[a:e].astype(np.float64), w[a:e].astype(np.float64), decreasing=dec)
            dev = float(np.max(np.abs(z[a:e] - zo) / (1 + np.abs(zo))))
            assert dev <= TOL[t], (r, e - a, dev)
