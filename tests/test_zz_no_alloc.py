"""iso_fit_noalloc: the fit with its workspace in the library's fixed device scratch.

Called through the C-ABI (ctypes) and compared bit for bit with iso_fit_ex given a workspace of
its own: the two run the same kernels, so z, block_start and row_flags must be identical.  Each
case makes two calls in a row, the second on a smaller input, so that the second call runs on
scratch the first one filled.
"""
import numpy as np
import pytest

from weighted_isotonic_regression_amd import binding as B
from weighted_isotonic_regression_amd import workloads as W

torch = pytest.importorskip("torch")


def _call_ex(y, w, flags):
    batch, n = y.shape
    code = B._dtype_code(torch, y)
    z = torch.empty_like(y)
    bs = torch.empty((batch, n), dtype=torch.uint8, device=y.device)
    rf = torch.empty((batch,), dtype=torch.int32, device=y.device)
    ws, nbytes = B.workspace(batch, n, code, w is not None, y.device)
    rc = B.iso_fit_ex(B._ptr(y), B._ptr(w), B._ptr(z), B._ptr(bs), B._ptr(rf), batch, n, code, B._ptr(ws), nbytes,
                      flags, B._stream(torch, y.device))
    assert rc == B.ISO_OK, B.iso_strerror(rc)
    return z, bs, rf


def _call_noalloc(y, w, flags, with_outputs=True):
    batch, n = y.shape
    code = B._dtype_code(torch, y)
    # poison the outputs so that a write that never happened shows
    z = torch.full_like(y, float("nan"))
    bs = torch.full((batch, n), 7, dtype=torch.uint8, device=y.device) if with_outputs else None
    rf = torch.full((batch,), -1, dtype=torch.int32, device=y.device) if with_outputs else None
    rc = B.iso_fit_noalloc(B._ptr(y), B._ptr(w), B._ptr(z), B._ptr(bs), B._ptr(rf), batch, n, code, flags,
                           B._stream(torch, y.device))
    assert rc == B.ISO_OK, B.iso_strerror(rc)
    return z, bs, rf


def _inputs(name, batch, n, seed, dtype, wkind):
    y, w = W.family(name, batch, n, seed=seed, dtype=dtype, wkind=wkind or "unit")
    yt = torch.from_numpy(np.ascontiguousarray(y)).cuda()
    wt = None if wkind is None else torch.from_numpy(np.ascontiguousarray(w)).cuda()
    return yt, wt


def _same(a, b):
    if a is None:
        return
    assert torch.equal(a.view(torch.uint8) if a.is_floating_point() else a,
                       b.view(torch.uint8) if b.is_floating_point() else b)


# (family, batch, n) of the first call, then of the second, smaller one
PAIRS = [
    (("noise", 2, 300_001), ("sawtooth", 3, 70_001)),       # long rows: chunks, scans and hull merges
    (("cancel", 1, 1_000_000), ("noise", 1, 20_000)),       # one long row, then a shorter one
    (("noise", 64, 5000), ("cliff", 5, 700)),               # rows of one or two waves
    (("noise", 4096, 16), ("constant", 100, 9)),            # short rows
]


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["f64", "f32"])
@pytest.mark.parametrize("weighted", [False, True])
@pytest.mark.parametrize("decreasing", [False, True])
@pytest.mark.parametrize("pair", range(len(PAIRS)))
def test_noalloc_matches_fit_ex(pair, dtype, weighted, decreasing):
    flags = B.ISO_FLAG_DECREASING if decreasing else 0
    for k, (fam, batch, n) in enumerate(PAIRS[pair]):
        print("noalloc case", pair, k, fam, batch, n, dtype, weighted, decreasing, flush=True)
        y, w = _inputs(fam, batch, n, 100 * pair + k, dtype, "extreme" if weighted else None)
        ref = _call_ex(y, w, flags)
        got = _call_noalloc(y, w, flags)
        torch.cuda.synchronize()
        assert not torch.isnan(got[0]).any()
        for a, b in zip(got, ref):
            _same(a, b)


@pytest.mark.gpu
def test_noalloc_without_optional_outputs_and_weight_check():
    # row_flags and block_start absent, weight check on: the row flags then live in the scratch
    y, w = _inputs("noise", 3, 200_000, 5, "f64", "extreme")
    ref = _call_ex(y, w, B.ISO_FLAG_CHECK_WEIGHTS)
    z, _, _ = _call_noalloc(y, w, B.ISO_FLAG_CHECK_WEIGHTS, with_outputs=False)
    _same(z, ref[0])
    y2, w2 = _inputs("sawtooth", 2, 50_000, 6, "f64", "extreme")
    w2[1, 17] = -1.0
    code = B._dtype_code(torch, y2)
    z2 = torch.empty_like(y2)
    rc = B.iso_fit_noalloc(B._ptr(y2), B._ptr(w2), B._ptr(z2), None, None, 2, 50_000, code,
                           B.ISO_FLAG_CHECK_WEIGHTS, B._stream(torch, y2.device))
    assert rc == B.ISO_EWEIGHT


@pytest.mark.gpu
def test_noalloc_rejects_oversize_before_launching():
    # one row of 1.5e8 elements needs more than the 256 MiB scratch; nothing is launched
    y = torch.zeros(16, dtype=torch.float64, device="cuda")
    z = torch.empty_like(y)
    n = 150_000_000
    assert B.iso_workspace_bytes(1, n, B.ISO_F64, 0) > B.ISO_NOALLOC_SCRATCH_BYTES
    rc = B.iso_fit_noalloc(B._ptr(y), None, B._ptr(z), None, None, 1, n, B.ISO_F64, 0,
                           B._stream(torch, y.device))
    assert rc == B.ISO_ESCRATCH
    assert "scratch" in B.iso_strerror(rc)
