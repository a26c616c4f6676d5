"""GPU parity of the one-row-per-workgroup kernel (1024 threads, the diagram in LDS,
candidate-parallel bridge searches), which fits rows of 2049 to 4096 elements and shorter rows in
batches of at most 256: every test family, weight kind, direction and element type against the
oracle (fp64 1e-10, fp32 1e-6, identical block starts where the partition is exact), rows that
start off 16-byte alignment, all-vertex rows, and batches.  Larger batches of rows of at most 2048
go to the packed short-row kernel, checked here too."""
import numpy as np
import pytest

import oracle
from weighted_isotonic_regression_amd import workloads as W

from tests.test_gpu_fit import check, gpu_fit, wrong_steps

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ROW_SIZES = (2049, 3001, 4095, 4096)


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("decreasing", [False, True])
@pytest.mark.parametrize("fam", W.FAMILIES)
def test_row_families(fam, decreasing, dtype):
    cancel = fam == "cancel"
    for n in ROW_SIZES:
        for wk in ("unit", "uniform", "integer", "extreme"):
            y, w = W.family(fam, 2, n, seed=n + 5, dtype=dtype, wkind=wk)
            w_ = None if wk == "unit" else w
            tol = (1.4e-15 if dtype == "f64" else 1e-7) if cancel else None
            exact = fam in ("integer", "constant") and wk in ("unit", "integer")
            z, _ = check(y, w_, exact_partition=exact, tol=tol, kkt=not cancel, scale_abs=cancel,
                         decreasing=decreasing)
            if wk == "extreme":
                assert wrong_steps(z, decreasing) <= 1e-15


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_row_all_vertices(dtype):
    """Strictly increasing rows: every point is a vertex, every merge keeps both hulls whole,
    and every element is its own block with z = y."""
    for n in (2049, 4096):
        y, w = W.family("increasing", 3, n, seed=1, dtype=dtype, wkind="uniform")
        for ww in (None, w):
            z, bs, rf = gpu_fit(y, ww)
            assert not rf.any() and bs.all()
            np.testing.assert_array_equal(z, y)


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_row_unaligned_start(dtype):
    """A row whose storage starts one element past a 16-byte boundary (scalar loads and
    stores), and rows of odd length packed back to back."""
    t = np.float32 if dtype == "f32" else np.float64
    rng = np.random.default_rng(4)
    n = 4093
    big = (np.arange(n + 1) / n + 0.3 * rng.standard_normal(n + 1)).astype(t)
    wbig = rng.uniform(0.5, 2.0, n + 1).astype(t)
    yt = torch.from_numpy(big).cuda()[1:]
    wt = torch.from_numpy(wbig).cuda()[1:]
    from weighted_isotonic_regression_amd import binding

    binding.load()
    z = binding.fit(yt, wt).cpu().numpy()
    zo = oracle.pav(big[1:].astype(np.float64), wbig[1:].astype(np.float64))
    assert np.max(np.abs(z.astype(np.float64) - zo) / (1 + np.abs(zo))) <= (1e-6 if dtype == "f32" else 1e-10)
    y, w = W.family("noise", 7, 3001, seed=9, dtype=dtype, wkind="uniform")
    check(y, w)


def test_row_config_ramp_batches():
    """The 4096-element ramp with noise, alone and in batches (one workgroup per row)."""
    for batch in (1, 2, 37, 300):
        y, w = W.ramp_noise_4096(batch=batch, seed=batch)
        check(y, w, exact_partition=False)


def test_row_integer_partitions_exact():
    for n in (2049, 2500, 4096):
        y, w = W.family("integer", 3, n, seed=n, dtype="f64", wkind="integer")
        check(y, w, exact_partition=True)
        y, w = W.calibration(seed=n, batch=2, n=n)
        check(y, w, exact_partition=True)


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("fam", W.FAMILIES)
def test_row_short_rows_small_batches(fam, dtype):
    """Rows of 17 to 2048 elements in batches of at most 256 (one workgroup per row, most threads
    without elements), both directions."""
    cancel = fam == "cancel"
    for n, batch in ((17, 1), (33, 256), (64, 5), (100, 3), (257, 2), (1000, 2), (2047, 1), (2048, 3)):
        for wk in ("unit", "uniform", "extreme"):
            y, w = W.family(fam, batch, n, seed=n + batch, dtype=dtype, wkind=wk)
            tol = (1.4e-15 if dtype == "f64" else 1e-7) if cancel else None
            exact = fam in ("integer", "constant") and wk == "unit"
            for dec in (False, True):
                check(y, None if wk == "unit" else w, exact_partition=exact, tol=tol, kkt=not cancel,
                      scale_abs=cancel, decreasing=dec)


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_packed_short_rows_large_batches(dtype):
    """Batches of more than 256 rows of 17 to 2048 elements: 64 / L rows packed per wavefront of the
    short-row kernel, a last wavefront partly filled."""
    for n, batch in ((17, 1000), (31, 257), (100, 300), (513, 301), (1000, 300), (2048, 257)):
        for fam, wk in (("noise", "uniform"), ("sawtooth", "unit"), ("integer", "integer")):
            y, w = W.family(fam, batch, n, seed=n, dtype=dtype, wkind=wk)
            check(y, None if wk == "unit" else w, exact_partition=fam == "integer")
            check(y, w, decreasing=True)


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_row_walk_fallback_matches_search(dtype):
    """The walk from the shared point, which the one-row kernel uses when rounding leaves its
    parallel bridge search inconclusive, forced for every bridge (ISO_FLAG_ROW_WALK): z and block
    starts bit for bit those of the parallel search on every family, and against the oracle."""
    from tests.test_gpu_fit import _gpu

    b = _gpu()
    tol = 1e-6 if dtype == "f32" else 1e-10
    for fam in W.FAMILIES:
        # bit for bit where no turn is near zero (integer and constant rows with integer weights,
        # whose sums and turns are exact; generic rows, where ties have probability zero); every
        # family against the oracle.  Equal neighbouring means with fractional weights make a turn
        # that is zero in exact arithmetic, which the two paths may round either way: z is the
        # same, the block start between the two blocks may not be.
        same = fam in ("noise", "sawtooth", "cliff", "integer", "constant", "increasing", "decreasing")
        wk = "integer" if fam in ("integer", "constant") else "uniform"
        for n, batch in ((17, 3), (1000, 2), (4096, 2)):
            y, w = W.family(fam, batch, n, seed=n + 11, dtype=dtype, wkind=wk)
            yt, wt = torch.from_numpy(y).cuda(), torch.from_numpy(w).cuda()
            for dec in (False, True):
                z1, b1 = b.fit(yt, wt, block_starts=True, decreasing=dec)
                z2, b2 = b.fit(yt, wt, block_starts=True, decreasing=dec, row_walk=True)
                torch.cuda.synchronize()
                z2 = z2.cpu().numpy()
                if same:
                    np.testing.assert_array_equal(z2, z1.cpu().numpy(), err_msg=f"{fam} {n} {dec}")
                    np.testing.assert_array_equal(b2.cpu().numpy(), b1.cpu().numpy())
                zo = oracle.pav(y.astype(np.float64), w.astype(np.float64), decreasing=dec).reshape(y.shape)
                if fam == "cancel":
                    dev = np.max(np.abs(z2.astype(np.float64) - zo)) / np.max(np.abs(y.astype(np.float64)))
                    assert dev <= (1.4e-15 if dtype == "f64" else 1e-7), (fam, n, dec, dev)
                else:
                    dev = np.max(np.abs(z2.astype(np.float64) - zo) / (1 + np.abs(zo)))
                    assert dev <= tol, (fam, n, dec, dev)
