"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws numbers: it holds none of the fit's arithmetic, so both the GPU path
and the CPU oracle can be fed from it without sharing code.  Every generator uses numpy's
PCG64 (``default_rng(seed)``), draws in fp64 and casts once to the requested dtype.

Workload families
-----------------
The named workloads are the five shapes the fit is measured on plus a dense 10^8 row:

``ramp_noise_4096``     1 x 4096 fp64, y_i = i/n + N(0, 0.3^2), w ~ U(0.5, 2.0)
``short_rows_16``       65536 x 16 fp32, y ~ N(0, 1), unit weights
``calibration``         512 x 131072 fp32, per row scores s ~ N(0,1) sorted ascending,
                        y ~ Bernoulli(sigmoid(1.5 s - 3)) in {0, 1}, w ~ U{1..4}
``nearly_monotone_1e7`` 1 x 10^7 fp64, y_i = i/n + N(0, (1e-9)^2), unit weights
``mixed_1e8``           1 x 10^8 fp32, y_i = sin(8 pi i/n) + 2 i/n + N(0, 0.05^2),
                        w ~ LogUniform[0.1, 10]
``nearly_monotone_1e8`` the nearly monotone generator at n = 10^8, fp64

The test families of "Merge Hulls Without Copying Vertices" (Section 7.1 and 7.6) are also
here: noise ramp, strictly increasing, sawtooth, cliff, constant, consecutive floats, the
cancellation family, integer-valued rows and extreme weights.  Where the page leaves a
family's parameters open (sawtooth period, cliff depth, the "extreme weights" distribution)
the choice made here is stated in the generator.
"""
from __future__ import annotations

import numpy as np

_DT = {"f32": np.float32, "f64": np.float64, np.float32: np.float32, np.float64: np.float64}


def _dt(dtype):
    if isinstance(dtype, str):
        return _DT[dtype]
    return np.dtype(dtype).type


def _index(n):
    return np.arange(n, dtype=np.float64)


# --------------------------------------------------------------------------- named workloads

def ramp_noise_4096(seed=1, n=4096, batch=1, dtype="f64"):
    """y_i = i/n + N(0, 0.3^2); w ~ U(0.5, 2.0)."""
    rng = np.random.default_rng(seed)
    t = _dt(dtype)
    y = _index(n)[None, :] / n + 0.3 * rng.standard_normal((batch, n))
    w = rng.uniform(0.5, 2.0, size=(batch, n))
    return y.astype(t), w.astype(t)


def short_rows_16(seed=2, batch=65536, n=16, dtype="f32"):
    """y ~ N(0, 1) i.i.d.; unit weights (returned as an explicit array of ones)."""
    rng = np.random.default_rng(seed)
    t = _dt(dtype)
    y = rng.standard_normal((batch, n))
    return y.astype(t), np.ones((batch, n), dtype=t)


def calibration(seed=3, batch=512, n=131072, dtype="f32"):
    """Calibration curves: sorted N(0,1) scores, Bernoulli(sigmoid(1.5 s - 3)) labels, integer
    weights in {1, 2, 3, 4} (downsampling weights).  Integer-valued, so exact partitions apply."""
    rng = np.random.default_rng(seed)
    t = _dt(dtype)
    y = np.empty((batch, n), dtype=t)
    w = np.empty((batch, n), dtype=t)
    for r in range(batch):
        s = np.sort(rng.standard_normal(n))
        p = 1.0 / (1.0 + np.exp(-(1.5 * s - 3.0)))
        y[r] = (rng.uniform(size=n) < p).astype(np.float64)
        w[r] = rng.integers(1, 5, size=n).astype(np.float64)
    return y, w


def nearly_monotone(seed=4, n=10_000_000, batch=1, dtype="f64", sigma=1e-9):
    """y_i = i/n + N(0, sigma^2), unit weights.  With sigma = 1e-9 every CSD point is a vertex."""
    rng = np.random.default_rng(seed)
    t = _dt(dtype)
    y = np.empty((batch, n), dtype=t)
    for r in range(batch):
        y[r] = (_index(n) / n + sigma * rng.standard_normal(n)).astype(t)
    return y, np.ones((batch, n), dtype=t)


def nearly_monotone_1e7(seed=4, n=10_000_000, dtype="f64"):
    return nearly_monotone(seed=seed, n=n, dtype=dtype)


def nearly_monotone_1e8(seed=6, n=100_000_000, dtype="f64"):
    return nearly_monotone(seed=seed, n=n, dtype=dtype)


def nearly_monotone_reversals_1e8(seed=8, n=100_000_000, dtype="f64"):
    """y_i = i/n + N(0, (2e-9)^2), unit weights: about one step in 5000 goes down (a few per
    16384-element chunk), so almost every CSD point is a vertex but nearly every chunk holds a
    reversal and takes the general chunk pass rather than the strictly increasing shortcut."""
    return nearly_monotone(seed=seed, n=n, dtype=dtype, sigma=2e-9)


def mixed_1e8(seed=5, n=100_000_000, batch=1, dtype="f32"):
    """y_i = sin(8 pi i/n) + 2 i/n + N(0, 0.05^2); w ~ LogUniform[0.1, 10]."""
    rng = np.random.default_rng(seed)
    t = _dt(dtype)
    y = np.empty((batch, n), dtype=t)
    w = np.empty((batch, n), dtype=t)
    for r in range(batch):
        i = _index(n)
        v = np.sin(8.0 * np.pi * i / n)
        v += 2.0 * i / n
        del i
        v += 0.05 * rng.standard_normal(n)
        y[r] = v.astype(t)
        del v
        w[r] = np.exp(rng.uniform(np.log(0.1), np.log(10.0), size=n)).astype(t)
    return y, w


def noise_1e7_decreasing(seed=7, n=10_000_000, dtype="f32"):
    """y ~ N(0, 1) i.i.d., one row, fp32, no weights (returned as None), to be fitted in the
    decreasing direction: the setting of the page's Table 1 comparison (Section 7.2), whose own
    inputs the page does not give."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((1, n)).astype(_dt(dtype)), None


WORKLOADS = {
    "ramp_noise_4096": ramp_noise_4096,
    "short_rows_16": short_rows_16,
    "calibration": calibration,
    "nearly_monotone_1e7": nearly_monotone_1e7,
    "mixed_1e8": mixed_1e8,
    "nearly_monotone_1e8": nearly_monotone_1e8,
    "nearly_monotone_reversals_1e8": nearly_monotone_reversals_1e8,
    "noise_1e7_decreasing": noise_1e7_decreasing,
}


# --------------------------------------------------------------------------- test families

def weights(rng, kind, shape, t):
    """Weight draws: 'unit', 'uniform' U(0.5, 2), 'extreme' LogUniform[1e-4, 1e4] (the page's
    'extreme weights' are not specified; this range is the choice made here), 'integer' U{1..4}."""
    if kind is None or kind == "unit":
        return np.ones(shape, dtype=t)
    if kind == "uniform":
        return rng.uniform(0.5, 2.0, size=shape).astype(t)
    if kind == "extreme":
        return np.exp(rng.uniform(np.log(1e-4), np.log(1e4), size=shape)).astype(t)
    if kind == "integer":
        return rng.integers(1, 5, size=shape).astype(t)
    raise ValueError(kind)


def family(name, batch, n, seed=0, dtype="f64", wkind="uniform"):
    """One test family as (y, w) of shape [batch, n].

    noise       ramp from 0 to 3 plus N(0, 1)
    increasing  strictly increasing: i/n plus a tiny positive jitter kept below the step
    sawtooth    ramps of period 3*2048 (rising 0 -> 5), so bridges reach across many chunks
    cliff       increasing values whose last element is -1e6
    constant    all values 1.5
    consecutive fp32/fp64 values each one ulp above the previous, starting at 1.0
    cancel      each 64 elements: 32 of +B, one of -32 B and 31 nearly collinear small values
                (B = 1e6)
    integer     values in {0, ..., 5}
    decreasing  strictly decreasing ramp (one block)
    """
    rng = np.random.default_rng(seed)
    t = _dt(dtype)
    i = _index(n)[None, :]
    shape = (batch, n)
    if name == "noise":
        y = 3.0 * i / max(n, 1) + rng.standard_normal(shape)
    elif name == "increasing":
        y = (i + 0.25 * rng.uniform(size=shape)) / max(n, 1)
    elif name == "sawtooth":
        period = 3 * 2048
        y = 5.0 * (i % period) / period + 0.01 * rng.standard_normal(shape)
    elif name == "cliff":
        y = np.broadcast_to(i / max(n, 1), shape).copy()
        y[:, -1] = -1e6
    elif name == "constant":
        y = np.full(shape, 1.5)
    elif name == "consecutive":
        start = t(1.0)
        row = np.empty(n, dtype=t)
        v = start
        for k in range(n):
            row[k] = v
            v = np.nextafter(v, t(np.inf))
        y = np.broadcast_to(row.astype(np.float64), shape).copy()
    elif name == "cancel":
        B = 1e6
        k = (i % 64)
        y = np.where(k < 32, B, np.where(k == 32, -32.0 * B, 1e-3 * (k - 33) + 1e-9 * rng.standard_normal(shape)))
        y = np.broadcast_to(y, shape).copy()
    elif name == "integer":
        y = rng.integers(0, 6, size=shape).astype(np.float64)
    elif name == "decreasing":
        y = np.broadcast_to(-i / max(n, 1), shape).copy()
    else:
        raise ValueError(name)
    return y.astype(t), weights(rng, wkind, shape, t)


FAMILIES = ("noise", "increasing", "sawtooth", "cliff", "constant", "consecutive", "cancel",
            "integer", "decreasing")
