"""GPU parity of rows of 2049 to 4096 elements, each fitted by one workgroup of 1024 threads with
the diagram in LDS and candidate-parallel bridge searches: every test family, weight kind,
direction and element type against the oracle (fp64 1e-10, fp32 1e-6, identical block starts
where the partition is exact), rows that start off 16-byte alignment, all-vertex rows, and
batches."""
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
