"""The oracle's pins are sharp: plausible mistakes planted in a copy of the oracle fail them.

Each case copies oracle/iso_oracle.c to a temporary directory, applies one textual mutation
(a dropped term, a wrong operand, a transposed comparison, an off-by-one, a non-canonical tie
rule), compiles it with gcc and runs a compact version of the pins of test_oracle.py against
it.  The unmutated copy must pass them and every mutant must fail at least one.  Everything
runs on the CPU; the real oracle is not touched.
"""
import ctypes
import os
import subprocess
import tempfile

import numpy as np
import pytest

from oracle import exact
from tests.test_oracle import GOLDEN_CASES

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "iso_oracle.c")

MUTANTS = {
    "strict_tie_rule": ("bs[top - 1] * bw[top] >= bs[top] * bw[top - 1]",
                        "bs[top - 1] * bw[top] > bs[top] * bw[top - 1]"),
    "dropped_weight_in_sum": ("bs[top] = wk * y[k];", "bs[top] = y[k];"),
    "wrong_operand_in_pool": ("bw[top - 1] += bw[top];", "bw[top - 1] += bs[top];"),
    "transposed_comparison": ("bs[top - 1] * bw[top] >= bs[top] * bw[top - 1]",
                              "bs[top - 1] * bw[top - 1] >= bs[top] * bw[top]"),
    "inverted_mean": ("double mean = bs[b] / bw[b];", "double mean = bw[b] / bs[b];"),
    "off_by_one_block_end": ("int64_t hi = (b < top) ? bstart[b + 1] : n;",
                             "int64_t hi = (b < top) ? bstart[b + 1] : n - 1;"),
    "pool_only_once": ("while (top >= 1 && (decreasing", "if (top >= 1 && (decreasing"),
    "decreasing_strict_tie_rule": ("bs[top - 1] * bw[top] <= bs[top] * bw[top - 1]",
                                   "bs[top - 1] * bw[top] < bs[top] * bw[top - 1]"),
    "decreasing_transposed_comparison": ("bs[top - 1] * bw[top] <= bs[top] * bw[top - 1]",
                                         "bs[top - 1] * bw[top - 1] <= bs[top] * bw[top]"),
    "direction_ignored": ("(decreasing ? ", "(0 ? "),
    "direction_not_passed": ("bs, decreasing);", "bs, 0);"),
    "wrong_sign_in_pool": ("bs[top - 1] += bs[top];", "bs[top - 1] -= bs[top];"),
}


def _build(src_text, tmp, name):
    c = os.path.join(tmp, name + ".c")
    so = os.path.join(tmp, name + ".so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-o", so, c, "-lm"],
                   check=True)
    lib = ctypes.CDLL(so)
    P = ctypes.c_void_p
    lib.iso_oracle_fit.argtypes = [P, P, P, P, P, ctypes.c_int64, ctypes.c_int64]
    lib.iso_oracle_fit.restype = ctypes.c_int
    lib.iso_oracle_fit_dir.argtypes = [P, P, P, P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
    lib.iso_oracle_fit_dir.restype = ctypes.c_int
    return lib


def _fit(lib, y, w, decreasing=False):
    y = np.ascontiguousarray(y, dtype=np.float64)[None, :]
    w = None if w is None else np.ascontiguousarray(w, dtype=np.float64)[None, :]
    z = np.empty_like(y)
    s = np.empty(y.shape, dtype=np.uint8)
    fl = np.empty(1, dtype=np.uint32)
    ptr = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    if decreasing:
        lib.iso_oracle_fit_dir(ptr(y), ptr(w), ptr(z), ptr(s), ptr(fl), 1, y.shape[1], 1)
    else:
        lib.iso_oracle_fit(ptr(y), ptr(w), ptr(z), ptr(s), ptr(fl), 1, y.shape[1])
    return z[0], s[0]


def _pins_pass(lib):
    """A compact run of the pins: golden rows, exact max-min / hull on random tiny rows, KKT,
    and the same for the decreasing direction against the exact min-max formula."""
    for y, w, z_exp, s_exp in GOLDEN_CASES:
        yf = np.array([float(v) for v in y])
        wf = None if w is None else np.array([float(v) for v in w])
        z, s = _fit(lib, yf, wf)
        if any(abs(a - float(b)) > 1e-15 * (1 + abs(float(b))) for a, b in zip(z, z_exp)):
            return False
        if list(s) != s_exp:
            return False
    rng = np.random.default_rng(99)
    for n in range(1, 11):
        for _ in range(4):
            y = rng.standard_normal(n)
            w = rng.uniform(0.2, 3.0, n)
            z, s = _fit(lib, y, w)
            zm = exact.maxmin(y, w)
            if any(abs(a - float(b)) > 1e-15 * (1 + abs(float(b))) for a, b in zip(z, zm)):
                return False
            if list(s) != exact.blocks_from_exact(zm):
                return False
            if exact.kkt_residual(y, w, z) > 1e-12:
                return False
            zd, sd = _fit(lib, y, w, decreasing=True)
            zx = exact.minmax(y, w)
            if any(abs(a - float(b)) > 1e-15 * (1 + abs(float(b))) for a, b in zip(zd, zx)):
                return False
            if list(sd) != exact.blocks_from_exact(zx):
                return False
            if exact.kkt_residual(y, w, zd, decreasing=True) > 1e-12:
                return False
            # ties: small integers, where the canonical rule decides the partition
            yi = rng.integers(0, 3, n).astype(float)
            wi = rng.integers(1, 4, n).astype(float)
            for dec, ex in ((False, exact.maxmin), (True, exact.minmax)):
                zt, st = _fit(lib, yi, wi, decreasing=dec)
                zx = ex(yi, wi)
                if any(a != float(b) for a, b in zip(zt, zx)) or list(st) != exact.blocks_from_exact(zx):
                    return False
    return True


def test_unmutated_copy_passes():
    with tempfile.TemporaryDirectory() as tmp:
        lib = _build(open(SRC).read(), tmp, "orig")
        assert _pins_pass(lib)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation site not found: %s" % name
    with tempfile.TemporaryDirectory() as tmp:
        lib = _build(text.replace(old, new), tmp, name)
        assert not _pins_pass(lib), "mutant %s survived the pins" % name
