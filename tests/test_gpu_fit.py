"""GPU parity: the HIP fit against the CPU oracle, element by element, through the C ABI.

Bars: max |z - z*| / (1 + |z*|) <= 1e-10 for fp64 and <= 1e-6 for fp32 (z* the oracle's fp64
fit of the same stored inputs); identical block starts on integer-valued inputs; every output
also passes the KKT certificate.  Sizes span several chunks of 2048 with ragged tails, and the
full measured shapes are run too.
"""
import numpy as np
import pytest

import oracle
from oracle import exact
from weighted_isotonic_regression_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {np.float32: 1e-6, np.float64: 1e-10}


def _gpu():
    from weighted_isotonic_regression_amd import binding

    binding.load()
    return binding


def gpu_fit(y, w, **kw):
    b = _gpu()
    yt = torch.from_numpy(np.ascontiguousarray(y)).cuda()
    wt = None if w is None else torch.from_numpy(np.ascontiguousarray(w)).cuda()
    res = b.fit(yt, wt, block_starts=True, row_flags=True, **kw)
    torch.cuda.synchronize()
    z, bs, rf = res
    return z.cpu().numpy(), bs.cpu().numpy(), rf.cpu().numpy()


def deviation(z, zo):
    z = z.astype(np.float64)
    return float(np.max(np.abs(z - zo) / (1 + np.abs(zo)))) if z.size else 0.0


def check(y, w, exact_partition=False, tol=None, kkt=True, scale_abs=False, decreasing=False):
    """scale_abs: measure max |z - z*| / max |y| instead (the page's Section 7.6 measure for its
    cancellation family, whose blocks mix values of very different sizes).  decreasing: fit and
    compare the non-increasing direction."""
    t = y.dtype.type
    z, bs, rf = gpu_fit(y, w, decreasing=decreasing)
    zo, bo, fo = oracle.pav(y.astype(np.float64), None if w is None else w.astype(np.float64),
                            return_blocks=True, decreasing=decreasing)
    zo = zo.reshape(y.shape)
    bo = bo.reshape(y.shape)
    assert np.array_equal(rf.astype(np.uint32), fo)
    if scale_abs:
        dev = float(np.max(np.abs(z.astype(np.float64) - zo)) / np.max(np.abs(y.astype(np.float64))))
    else:
        dev = deviation(z, zo)
    assert dev <= (tol or TOL[t]), dev
    if exact_partition:
        assert np.array_equal(bs, bo)
    if kkt and y.ndim == 2 and y.shape[1] <= 300_000:
        for r in range(min(y.shape[0], 3)):
            assert exact.kkt_residual(y[r], None if w is None else w[r], z[r], decreasing=decreasing) < (
                1e-12 if t == np.float64 else 1e-6)
    return z, bs


SIZES = [1, 2, 3, 17, 31, 32, 33, 63, 64, 65, 100, 511, 1000, 1024, 1025, 2047, 2048, 2049, 4095, 4096,
         4097, 6145, 8191, 8192, 8193, 10000, 16383, 16384, 16385, 49153, 65536, 100003, 200001]


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("n", SIZES)
def test_noise_sizes(n, dtype):
    batch = 3 if n < 100000 else 1
    for wk in ("unit", "uniform"):
        y, w = W.family("noise", batch, n, seed=n, dtype=dtype, wkind=wk)
        check(y, None if wk == "unit" else w)


@pytest.mark.parametrize("fam", W.FAMILIES)
@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_families(fam, dtype):
    for n in (700, 5000, 70001):
        for wk in ("unit", "uniform", "integer"):
            y, w = W.family(fam, 2, n, seed=n + 1, dtype=dtype, wkind=wk)
            w_ = None if wk == "unit" else w
            # The cancellation family is measured against max|y| (the page's Section 7.6 does so),
            # to the page's fp64 figure, 1.4e-15 max|y|; fp32 outputs carry their own rounding,
            # up to 6e-8 of |z| <= max|y|.
            cancel = fam == "cancel"
            tol = (1.4e-15 if dtype == "f64" else 1e-7) if cancel else None
            check(y, w_, exact_partition=(fam in ("integer", "constant") and wk != "uniform"), tol=tol,
                  kkt=not cancel, scale_abs=cancel)


@pytest.mark.parametrize("n", [5, 64, 2048, 2049, 40000])
def test_integer_partitions_exact(n):
    y, w = W.family("integer", 4, n, seed=3, dtype="f32", wkind="integer")
    check(y, w, exact_partition=True)
    y, w = W.calibration(seed=9, batch=2, n=n)
    check(y, w, exact_partition=True)


def test_config_ramp_noise_4096():
    y, w = W.ramp_noise_4096()
    check(y, w)
    check(y, None)


def test_config_short_rows_16():
    y, w = W.short_rows_16()
    check(y, w)
    check(y, None)


def test_config_calibration_full():
    y, w = W.calibration()
    check(y, w, exact_partition=True, kkt=False)


def test_config_nearly_monotone_1e7():
    y, w = W.nearly_monotone_1e7()
    assert np.all(np.diff(y[0]) > 0)
    for ww in (w, None):
        z, bs = check(y, ww, kkt=False)
        assert bs.all()  # every element its own block


def test_config_mixed_1e8():
    y, w = W.mixed_1e8()
    check(y, w, kkt=False)


def test_nearly_monotone_1e8_fp64():
    y, w = W.nearly_monotone_1e8()
    for ww in (None, w):
        z, bs = check(y, ww, kkt=False)
        assert bs.all()
        np.testing.assert_array_equal(z, y)  # one-element blocks output their y


def test_nearly_monotone_reversals_1e8_fp64():
    """The dense hull through the general chunk pass: a few reversals in nearly every chunk of
    16384, so the strictly increasing shortcut rarely applies and almost every point is a
    vertex.  Against the oracle at 1e-10, block starts identical (every block boundary here is
    decided by steps of about 1e-8 against noise of 2e-9, far from any tie)."""
    y, w = W.nearly_monotone_reversals_1e8()
    chunks = y[0, : (y.shape[1] // 16384) * 16384].reshape(-1, 16384)
    assert np.mean(np.any(np.diff(chunks, axis=1) <= 0, axis=1)) > 0.9
    for ww in (w, None):
        z, bs = check(y, ww, kkt=False, exact_partition=True)
        assert bs.mean() > 0.99


def wrong_steps(z, decreasing=False):
    """Largest step of z against the fit direction, relative to max(1, max |z|)."""
    z = np.asarray(z, dtype=np.float64)
    steps = np.diff(z, axis=-1)
    worst = float(np.max(steps if decreasing else -steps, initial=0.0))
    return max(worst, 0.0) / max(1.0, float(np.max(np.abs(z))))


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("decreasing", [False, True])
@pytest.mark.parametrize("fam", W.FAMILIES)
def test_extreme_weights(fam, decreasing, dtype):
    """Weights spanning eight orders of magnitude (LogUniform[1e-4, 1e4], the page's "extreme
    weights" of Section 7.6) on every family and size class: the fp64 bar 1e-10 and fp32 1e-6 (the
    cancellation family against max |y| at the page's fp64 figure 1.4e-15), the KKT certificate,
    and no step against the fit direction beyond a few units in the last place.  Slopes of short
    edges over tiny weights are differences of prefix sums many orders larger, so these rows need
    the coordinate pairs and the filtered predicates."""
    cancel = fam == "cancel"
    for n in (700, 5000, 70001, 1_000_000):
        y, w = W.family(fam, 2 if n < 100000 else 1, n, seed=n + 17, dtype=dtype, wkind="extreme")
        tol = (1.4e-15 if dtype == "f64" else 1e-7) if cancel else None
        z, bs = check(y, w, tol=tol, kkt=not cancel, scale_abs=cancel, decreasing=decreasing)
        assert wrong_steps(z, decreasing) <= 1e-15, (n, wrong_steps(z, decreasing))


def test_page_stress_row_increasing_extreme_weights_1e7():
    """The page's Section 7.6 stress case: 10^7 strictly increasing fp64 values with extreme
    weights, whose cumulative sums reach about 10^10.  Every point is a vertex of the exact hull,
    so every element is its own block and the fit is y itself; the page reports that a version
    without the coordinate hierarchy pools 681 of these points."""
    y, w = W.family("increasing", 1, 10_000_000, seed=11, dtype="f64", wkind="extreme")
    assert np.all(np.diff(y[0]) > 0)
    z, bs, rf = gpu_fit(y, w)
    assert rf[0] == 0
    assert bs.all()
    np.testing.assert_array_equal(z, y)
    # the same row with reversals every few hundred elements: most points stay vertices
    yr = y.copy()
    yr[0, 300::977] -= 3e-6
    z, bs = check(yr, w, kkt=False)
    assert wrong_steps(z) <= 1e-15


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_increasing_chunks_with_one_break(dtype):
    """Rows that are strictly increasing except at one element: a tie or a drop at the first,
    middle or last element of a full 16384-element chunk (a chunk that is increasing throughout
    is a whole-diagram hull; one that breaks late is processed again by the lane chains), and a
    drop deep enough to pool across several increasing chunks."""
    C = 16384
    n = 3 * C + 100
    t = np.float32 if dtype == "f32" else np.float64
    base = np.arange(n, dtype=np.float64) / n
    cases = [(C, "tie"), (C + C // 2 - 1, "drop"), (2 * C - 1, "tie"), (3 * C - 1, "drop"), (C - 1, "drop"),
             (2 * C + 5, "cliff")]
    rows = []
    for pos, kind in cases:
        y = base.copy()
        if kind == "tie":
            y[pos] = y[pos - 1]
        elif kind == "drop":
            y[pos] = y[pos - 1] - 1e-3
        else:
            y[pos] = -5.0
        rows.append(y)
    y = np.stack(rows).astype(t)
    rng = np.random.default_rng(11)
    w = rng.uniform(0.5, 2.0, size=y.shape).astype(t)
    check(y, w)
    check(y, None)


def test_increasing_row_with_nan_is_flagged():
    n = 2 * 16384
    y = np.tile(np.arange(n, dtype=np.float64) / n, (2, 1))
    y[1, 20000] = np.nan
    z, bs, flags = gpu_fit(y, None)
    assert flags[0] == 0 and flags[1] == 1
    assert np.isnan(z[1]).all()
    np.testing.assert_array_equal(z[0], y[0])
    assert bs[0].all()


def test_row_of_8194_chunks():
    """A row of more than 8192 chunks of 16384 (over 1.34e8 elements, eight scan blocks)."""
    n = 8193 * 16384 + 77
    y, w = W.family("noise", 1, n, seed=21, dtype="f32", wkind="uniform")
    check(y, w, kkt=False)


@pytest.mark.parametrize("chunks", [9, 17, 65])
def test_batched_rows_of_several_merge_subtrees(chunks):
    """Batches of rows of 9, 17 and 65 chunks, the last one ragged.  The merge tree of such a row
    has 4, 5 and 7 levels, so its levels do not split evenly into groups of three, and its first
    group holds 2, 3 and 9 subtrees of eight chunks.  Every row must be merged from its own
    chunks.  Three families are run: the mixed trend (long walks at the upper levels), noise, and
    integers (whose partition must match exactly)."""
    n = (chunks - 1) * 16384 + 1001
    y, w = W.mixed_1e8(seed=chunks, n=n, batch=3)
    check(y, w, kkt=False)
    y, w = W.family("noise", 3, n, seed=chunks, dtype="f64", wkind="uniform")
    check(y, w, kkt=False)
    y, w = W.family("integer", 3, n, seed=chunks, dtype="f32", wkind="integer")
    check(y, w, exact_partition=True, kkt=False)


def test_65537_long_rows():
    """A batch of 65537 rows of 2049 (long rows, one chunk each): more rows than a grid's second
    dimension holds."""
    y, w = W.family("noise", 65537, 2049, seed=22, dtype="f32", wkind="uniform")
    check(y, w, kkt=False)


def test_bad_rows_flagged_and_others_fitted():
    b = _gpu()
    for n in (10, 3000):
        y, w = W.family("noise", 5, n, seed=2, dtype="f64", wkind="uniform")
        y[1, n // 2] = np.nan
        w[3, n - 1] = -1.0
        w[4, 0] = np.inf
        z, bs, rf = gpu_fit(y, w)
        assert list(rf) == [0, b.ISO_ROW_NONFINITE, 0, b.ISO_ROW_BAD_WEIGHT, b.ISO_ROW_NONFINITE]
        for r in (1, 3, 4):
            assert np.all(np.isnan(z[r])) and bs[r].sum() == 0
        for r in (0, 2):
            assert deviation(z[r], oracle.pav(y[r], w[r])) <= 1e-10
        yt = torch.from_numpy(y).cuda()
        wt = torch.from_numpy(w).cuda()
        with pytest.raises(b.IsoError) as ei:
            b.fit(yt, wt, check_weights=True)
        assert ei.value.code == b.ISO_EWEIGHT
        # through the simple entry point: weighted calls check
        zt = torch.empty_like(yt)
        import ctypes

        rc = b.iso_fit(ctypes.c_void_p(yt.data_ptr()), ctypes.c_void_p(wt.data_ptr()),
                       ctypes.c_void_p(zt.data_ptr()), 5, n, b.ISO_F64,
                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert rc == b.ISO_EWEIGHT


def test_simple_entry_point_matches():
    import ctypes

    b = _gpu()
    for n in (16, 5000):
        y, w = W.family("sawtooth", 3, n, seed=4, dtype="f32", wkind="uniform")
        yt, wt = torch.from_numpy(y).cuda(), torch.from_numpy(w).cuda()
        zt = torch.empty_like(yt)
        rc = b.iso_fit(ctypes.c_void_p(yt.data_ptr()), ctypes.c_void_p(wt.data_ptr()),
                       ctypes.c_void_p(zt.data_ptr()), 3, n, b.ISO_F32,
                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert rc == 0
        torch.cuda.synchronize()
        z2 = b.fit(yt, wt)
        assert torch.equal(zt, z2)


def test_deterministic_repeat():
    b = _gpu()
    y, w = W.family("sawtooth", 2, 300000, seed=5, dtype="f64", wkind="uniform")
    yt, wt = torch.from_numpy(y).cuda(), torch.from_numpy(w).cuda()
    z1, s1 = b.fit(yt, wt, block_starts=True)
    z2, s2 = b.fit(yt, wt, block_starts=True)
    assert torch.equal(z1, z2) and torch.equal(s1, s2)


def test_empty_and_tiny():
    b = _gpu()
    y = torch.empty((0, 7), dtype=torch.float32, device="cuda")
    assert b.fit(y).shape == (0, 7)
    y = torch.empty((3, 0), dtype=torch.float64, device="cuda")
    assert b.fit(y).shape == (3, 0)
    y = torch.tensor([[2.5], [-1.0]], dtype=torch.float64, device="cuda")
    assert torch.equal(b.fit(y), y)


@pytest.mark.parametrize("n", [1000, 2048, 20001, 70000])
def test_one_element_blocks_output_their_y(n):
    """A block of one element gets its y, its exact mean: on a ramp through zero from -1e20 to 1e20,
    where the diagram's coordinates are twenty orders of magnitude above the elements near zero,
    and on a noisy trend, whose long rows are chunks of both storage forms with one-element blocks
    inside them and at their ends; short rows, both directions, both dtypes."""
    for dtype in (np.float32, np.float64):
        y = np.linspace(-1e20, 1e20, n).astype(dtype)[None, :]
        z, bs, rf = gpu_fit(y, None)
        assert bs.all()
        np.testing.assert_array_equal(z, y)
        rng = np.random.default_rng(n)
        base = (np.arange(n) * 1e-3 + 1e-3 * rng.standard_normal((4, n))).astype(dtype)
        w2 = rng.uniform(0.5, 2.0, (4, n)).astype(dtype)
        for dec in (False, True):
            y2 = -base if dec else base  # a noisy trend in the fitted direction: blocks of all sizes
            z2, bs2, _ = gpu_fit(y2, w2, decreasing=dec)
            ends = np.concatenate([bs2[:, 1:], np.ones((4, 1), dtype=bs2.dtype)], axis=1)
            one = (bs2 == 1) & (ends == 1)
            assert one.sum() > 0
            np.testing.assert_array_equal(z2[one], y2[one])


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_tiny_rows_every_length(dtype):
    """Rows of 1 to 16 elements (one lane per row, pool adjacent violators): every length, with and
    without weights, both directions, batches that do and do not fill the last wavefront, exact
    partitions on integer rows."""
    for n in range(1, 17):
        for batch in (1, 63, 200):
            y, w = W.family("noise", batch, n, seed=n * 7 + batch, dtype=dtype, wkind="uniform")
            for dec in (False, True):
                check(y, w, decreasing=dec)
                check(y, None, decreasing=dec)
        yi, wi = W.family("integer", 130, n, seed=n, dtype=dtype, wkind="integer")
        for dec in (False, True):
            check(yi, wi, exact_partition=True, decreasing=dec)


def test_tiny_rows_flags_and_ties():
    b = _gpu()
    y = np.array([[1.0, 1.0, 1.0, 0.0], [2.0, np.nan, 1.0, 0.0], [3.0, 1.0, 2.0, 2.0], [0.0, 5.0, 5.0, 1.0]])
    w = np.array([[1.0, 2.0, 1.0, 1.0], [1.0, 1.0, 1.0, 1.0], [1.0, 1.0, -1.0, 1.0], [1.0, 1.0, 1.0, 1.0]])
    z, bs, rf = gpu_fit(y, w)
    assert list(rf) == [0, b.ISO_ROW_NONFINITE, b.ISO_ROW_BAD_WEIGHT, 0]
    assert np.isnan(z[1:3]).all() and bs[1:3].sum() == 0
    np.testing.assert_array_equal(z[0], [0.8, 0.8, 0.8, 0.8])
    np.testing.assert_array_equal(bs[0], [1, 0, 0, 0])
    np.testing.assert_array_equal(z[3], [0.0, 11.0 / 3, 11.0 / 3, 11.0 / 3])
    np.testing.assert_array_equal(bs[3], [1, 1, 0, 0])


def test_rare_branches_run_and_stay_exact():
    """The branches that only degenerate or far-reaching diagrams take, each shown to run (through
    iso_prof_counters) on a row whose fit is then checked against the oracle:
    - a cliff (a ramp whose last element is -1e6) pulls the top merge's bridge back over the whole
      first half, past 32 memory windows, onto the Overmars-van Leeuwen bisection;
    - sawtooth ramps make merges walk in memory windows;
    - y alternating 0.5, 1.5 with weights 0.25, 0.75: the candidate points (each 1.5 after a 0.5)
      are exactly collinear and every sum is exact, so the chain's turns are exactly zero, inside
      their error bounds, and the exact chunk pass decides them.  The fit is 0.5 for the first
      element and 1.25 (one pooled block) for the rest."""
    b = _gpu()
    b.iso_prof_counters(reset=True)
    y, w = W.family("cliff", 1, 1 << 20, seed=3, dtype="f64", wkind="uniform")
    check(y, w, kkt=False)
    c = b.iso_prof_counters(reset=True)
    assert c["bisections"] >= 1, c
    assert c["memory_window_merges"] >= 1, c
    y, w = W.family("sawtooth", 1, 1 << 20, seed=4, dtype="f32", wkind="unit")
    check(y, w, kkt=False)
    c = b.iso_prof_counters(reset=True)
    assert c["memory_window_merges"] >= 1, c
    n = 70001
    y = np.where(np.arange(n) % 2 == 0, 0.5, 1.5).reshape(1, n)
    w = np.where(np.arange(n) % 2 == 0, 0.25, 0.75).reshape(1, n)
    z, _ = check(y, w, exact_partition=True)
    c = b.iso_prof_counters(reset=True)
    assert c["exact_pass_chunks"] >= 1, c
    assert z[0, 0] == 0.5 and np.all(z[0, 1:] == 1.25)
