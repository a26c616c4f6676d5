"""Thin ctypes binding of the C ABI in include/iso.h (argument marshalling only).

The raw functions keep the C names and signatures (device pointers as ints, stream as an
int handle).  ``fit`` and ``vjp`` marshal torch tensors: they check shapes, dtypes and
devices, allocate outputs and the workspace with torch, and pass torch's current stream.
Every step of the fit runs in the HIP library; if the library is not built, or no GPU is
present, these functions raise.
"""
from __future__ import annotations

import ctypes
import os
import threading

from . import build as _build

ISO_F32, ISO_F64 = 0, 1
ISO_OK, ISO_EINVAL, ISO_EWEIGHT, ISO_ENOMEM, ISO_EHIP, ISO_ESCRATCH = 0, 1, 2, 3, 4, 5
ISO_NOALLOC_SCRATCH_BYTES = 256 << 20
ISO_FLAG_CHECK_WEIGHTS = 1
ISO_FLAG_DECREASING = 2
ISO_FLAG_ROW_WALK = 4
ISO_ROW_NONFINITE, ISO_ROW_BAD_WEIGHT = 1, 2

_lock = threading.Lock()
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SIGS = {
    "iso_fit": ([_P, _P, _P, _I64, _I64, ctypes.c_int, _P], ctypes.c_int),
    "iso_workspace_bytes": ([_I64, _I64, ctypes.c_int, ctypes.c_int], ctypes.c_size_t),
    "iso_fit_ex": ([_P, _P, _P, _P, _P, _I64, _I64, ctypes.c_int, _P, ctypes.c_size_t, ctypes.c_uint, _P],
                   ctypes.c_int),
    "iso_fit_noalloc": ([_P, _P, _P, _P, _P, _I64, _I64, ctypes.c_int, ctypes.c_uint, _P], ctypes.c_int),
    "iso_vjp": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I64, ctypes.c_int, _P], ctypes.c_int),
    "iso_fit_ragged": ([_P, _P, _P, _I64, ctypes.c_int, _P, _P, _P, _P, ctypes.c_size_t, ctypes.c_uint, _P],
                       ctypes.c_int),
    "iso_ragged_workspace_bytes": ([_P, _I64, ctypes.c_int, ctypes.c_int], ctypes.c_size_t),
    "iso_soft_rank": ([_P, _I64, _I64, ctypes.c_int, ctypes.c_double, _P, _P, _P, _P, _P], ctypes.c_int),
    "iso_soft_rank_vjp": ([_P, _P, _P, _I64, _I64, ctypes.c_int, ctypes.c_double, _P, _P], ctypes.c_int),
    "iso_strerror": ([ctypes.c_int], ctypes.c_char_p),
    "iso_prof_enable": ([ctypes.c_int], ctypes.c_int),
    "iso_prof_read": ([_P, _P, _P], ctypes.c_int),
    "iso_prof_stage_name": ([ctypes.c_int], ctypes.c_char_p),
    "iso_prof_counters": ([_P, ctypes.c_int], ctypes.c_int),
}
ISO_PROF_STAGES = 7
ISO_PROF_COUNTERS = 4
PROF_COUNTER_NAMES = ("bisections", "bisections_finished_by_steps", "exact_pass_chunks", "memory_window_merges")


class IsoError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__("%s failed: %s (code %d)" % (where, iso_strerror(code), code))


def library_path() -> str:
    return _build.LIB


def load():
    """Load libiso_mi355x.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            path = library_path()
            if not os.path.exists(path):
                raise RuntimeError("the HIP library %s is not built; run __graft_entry__.build()" % path)
            lib = ctypes.CDLL(path)
            for name, (args, res) in _SIGS.items():
                fn = getattr(lib, name)
                fn.argtypes = args
                fn.restype = res
            _lib = lib
    return _lib


# ------------------------------------------------------------------ raw C ABI

def iso_fit(y, w, z, batch, n, dtype, stream):
    return load().iso_fit(y, w, z, batch, n, dtype, stream)


def iso_workspace_bytes(batch, n, dtype, weighted):
    return load().iso_workspace_bytes(batch, n, dtype, int(bool(weighted)))


def iso_fit_ex(y, w, z, block_start, row_flags, batch, n, dtype, ws, ws_bytes, flags, stream):
    return load().iso_fit_ex(y, w, z, block_start, row_flags, batch, n, dtype, ws, ws_bytes, flags, stream)


def iso_fit_noalloc(y, w, z, block_start, row_flags, batch, n, dtype, flags, stream):
    return load().iso_fit_noalloc(y, w, z, block_start, row_flags, batch, n, dtype, flags, stream)


def iso_vjp(g, y, w, z, block_start, gy, gw, batch, n, dtype, stream):
    return load().iso_vjp(g, y, w, z, block_start, gy, gw, batch, n, dtype, stream)


def iso_fit_ragged(values, weights, offsets, batch, dtype, z, block_start, row_flags, ws, ws_bytes, flags, stream):
    return load().iso_fit_ragged(values, weights, offsets, batch, dtype, z, block_start, row_flags, ws, ws_bytes,
                                 flags, stream)


def iso_ragged_workspace_bytes(offsets, batch, dtype, weighted):
    return load().iso_ragged_workspace_bytes(offsets, batch, dtype, int(bool(weighted)))


def iso_soft_rank(x, batch, n, dtype, eps, r, perm, block_start, row_flags, stream):
    return load().iso_soft_rank(x, batch, n, dtype, eps, r, perm, block_start, row_flags, stream)


def iso_soft_rank_vjp(g, perm, block_start, batch, n, dtype, eps, grad, stream):
    return load().iso_soft_rank_vjp(g, perm, block_start, batch, n, dtype, eps, grad, stream)


def iso_strerror(code):
    return load().iso_strerror(code).decode()


def iso_prof_enable(on):
    return load().iso_prof_enable(int(bool(on)))


def iso_prof_read():
    """Returns ({stage name: ms}, {stage name: launches}, calls) accumulated since the last read."""
    ms = (ctypes.c_double * ISO_PROF_STAGES)()
    la = (ctypes.c_int64 * ISO_PROF_STAGES)()
    calls = ctypes.c_int64(0)
    rc = load().iso_prof_read(ms, la, ctypes.byref(calls))
    if rc != ISO_OK:
        raise IsoError(rc, "iso_prof_read")
    names = [load().iso_prof_stage_name(k).decode() for k in range(ISO_PROF_STAGES)]
    return dict(zip(names, list(ms))), dict(zip(names, list(la))), calls.value


def iso_prof_counters(reset=True):
    """Counts of rarely taken branches since the last reset, as {name: count} (waits for the device)."""
    out = (ctypes.c_uint64 * ISO_PROF_COUNTERS)()
    rc = load().iso_prof_counters(out, int(bool(reset)))
    if rc != ISO_OK:
        raise IsoError(rc, "iso_prof_counters")
    return dict(zip(PROF_COUNTER_NAMES, list(out)))


# ------------------------------------------------------------------ torch marshalling

def _torch():
    import torch

    if not torch.cuda.is_available():
        raise RuntimeError("no GPU: the isotonic fit runs only on the HIP device")
    return torch


def _dtype_code(torch, t):
    if t.dtype == torch.float32:
        return ISO_F32
    if t.dtype == torch.float64:
        return ISO_F64
    raise TypeError("y must be float32 or float64")


def _as_rows(t):
    if t.dim() == 1:
        return t.reshape(1, -1)
    if t.dim() != 2:
        raise ValueError("expected a row [n] or a batch of rows [batch, n]")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(torch, device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def workspace(batch, n, dtype_code, weighted, device):
    """A torch uint8 buffer of iso_workspace_bytes, 256-byte aligned (None if none is needed)."""
    torch = _torch()
    nbytes = iso_workspace_bytes(batch, n, dtype_code, weighted)
    if nbytes == 0:
        return None, 0
    buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    shift = (-buf.data_ptr()) % 256
    return buf[shift:shift + nbytes], nbytes


def fit(y, w=None, *, block_starts=False, row_flags=False, check_weights=False, decreasing=False, out=None,
        ws=None, row_walk=False):
    """Isotonic weighted L2 fit of every row of ``y`` on its device: non-decreasing, or
    non-increasing with ``decreasing=True``.

    y: float32/float64 CUDA tensor [n] or [batch, n]; w: same shape and dtype, or None.
    row_walk (testing): ISO_FLAG_ROW_WALK, bridges of the one-row kernel found by the walk.
    Returns z, or (z, block_start[uint8], row_flags[int32]) as requested.
    """
    torch = _torch()
    y2 = _as_rows(y)
    if not y2.is_cuda or not y2.is_contiguous():
        raise ValueError("y must be a contiguous tensor on the GPU")
    code = _dtype_code(torch, y2)
    w2 = None
    if w is not None:
        w2 = _as_rows(w)
        if w2.shape != y2.shape or w2.dtype != y2.dtype or w2.device != y2.device or not w2.is_contiguous():
            raise ValueError("w must be a contiguous tensor of y's shape, dtype and device")
    batch, n = y2.shape
    z = torch.empty_like(y2) if out is None else _as_rows(out)
    bs = torch.empty((batch, n), dtype=torch.uint8, device=y2.device) if block_starts else None
    rf = torch.empty((batch,), dtype=torch.int32, device=y2.device) if row_flags else None
    if ws is None:
        ws, nbytes = workspace(batch, n, code, w2 is not None, y2.device)
    else:
        nbytes = ws.numel()
    flags = (ISO_FLAG_CHECK_WEIGHTS if check_weights else 0) | (ISO_FLAG_DECREASING if decreasing else 0)
    if row_walk:  # testing: ISO_FLAG_ROW_WALK
        flags |= ISO_FLAG_ROW_WALK
    rc = iso_fit_ex(_ptr(y2), _ptr(w2), _ptr(z), _ptr(bs), _ptr(rf), batch, n, code, _ptr(ws), nbytes, flags,
                    _stream(torch, y2.device))
    if rc != ISO_OK:
        raise IsoError(rc, "iso_fit_ex")
    z = z.reshape(y.shape)
    if not block_starts and not row_flags:
        return z
    res = [z]
    if block_starts:
        res.append(bs.reshape(y.shape))
    if row_flags:
        res.append(rf)
    return tuple(res)


def fit_ragged(values, offsets, weights=None, *, decreasing=False, block_starts=False, row_flags=False,
               check_weights=False):
    """Fit rows of unequal lengths laid end to end: row r is values[offsets[r]:offsets[r + 1]].

    values, weights: 1-D float32/float64 CUDA tensors (weights may be None); offsets: batch + 1
    non-decreasing integers on the host (a list, numpy array or CPU tensor).  Returns z (same
    layout as values), or (z, block_start[uint8], row_flags[int32]) as requested.
    """
    import numpy as np

    torch = _torch()
    if values.dim() != 1 or not values.is_cuda or not values.is_contiguous():
        raise ValueError("values must be a contiguous 1-D tensor on the GPU")
    code = _dtype_code(torch, values)
    if weights is not None and (weights.shape != values.shape or weights.dtype != values.dtype or
                                weights.device != values.device or not weights.is_contiguous()):
        raise ValueError("weights must be a contiguous tensor of values' shape, dtype and device")
    offs = np.ascontiguousarray(np.asarray(offsets.cpu() if hasattr(offsets, "cpu") else offsets, dtype=np.int64))
    batch = offs.size - 1
    if batch < 0 or (batch > 0 and offs[-1] > values.numel()):
        raise ValueError("offsets must hold batch + 1 entries within values")
    op = offs.ctypes.data_as(ctypes.c_void_p)
    z = torch.empty_like(values)
    bs = torch.empty(values.shape, dtype=torch.uint8, device=values.device) if block_starts else None
    rf = torch.empty((max(batch, 0),), dtype=torch.int32, device=values.device) if row_flags else None
    nbytes = iso_ragged_workspace_bytes(op, batch, code, weights is not None)
    ws = None
    if nbytes:
        buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=values.device)
        shift = (-buf.data_ptr()) % 256
        ws = buf[shift:shift + nbytes]
    flags = (ISO_FLAG_CHECK_WEIGHTS if check_weights else 0) | (ISO_FLAG_DECREASING if decreasing else 0)
    rc = iso_fit_ragged(_ptr(values), _ptr(weights), op, batch, code, _ptr(z), _ptr(bs), _ptr(rf), _ptr(ws), nbytes,
                        flags, _stream(torch, values.device))
    if rc != ISO_OK:
        raise IsoError(rc, "iso_fit_ragged")
    if not block_starts and not row_flags:
        return z
    res = [z]
    if block_starts:
        res.append(bs)
    if row_flags:
        res.append(rf)
    return tuple(res)


def soft_rank(x, eps, *, row_flags=False):
    """Soft ranks of every row of x (float32/float64 CUDA tensor [n] or [batch, n]) with L2
    regularization of strength eps.  Returns (r, perm, block_start) -- perm (int32 tensor holding
    the uint32 sort permutation) and block_start are what soft_rank_vjp needs -- and the per-row
    flags too when row_flags is set."""
    torch = _torch()
    x2 = _as_rows(x)
    if not x2.is_cuda or not x2.is_contiguous():
        raise ValueError("x must be a contiguous tensor on the GPU")
    code = _dtype_code(torch, x2)
    batch, n = x2.shape
    r = torch.empty_like(x2)
    perm = torch.empty((batch, n), dtype=torch.int32, device=x2.device)
    bs = torch.empty((batch, n), dtype=torch.uint8, device=x2.device)
    rf = torch.empty((batch,), dtype=torch.int32, device=x2.device) if row_flags else None
    rc = iso_soft_rank(_ptr(x2), batch, n, code, float(eps), _ptr(r), _ptr(perm), _ptr(bs), _ptr(rf),
                       _stream(torch, x2.device))
    if rc != ISO_OK:
        raise IsoError(rc, "iso_soft_rank")
    res = (r.reshape(x.shape), perm, bs)
    return res + (rf,) if row_flags else res


def soft_rank_vjp(g, perm, block_start, eps):
    """Cotangent of x for the cotangent g of soft_rank's r."""
    torch = _torch()
    g2 = _as_rows(g)
    code = _dtype_code(torch, g2)
    batch, n = g2.shape
    if perm.shape != (batch, n) or block_start.shape != (batch, n) or not g2.is_contiguous():
        raise ValueError("perm and block_start must come from soft_rank of x of g's shape")
    grad = torch.empty_like(g2)
    rc = iso_soft_rank_vjp(_ptr(g2), _ptr(perm), _ptr(block_start), batch, n, code, float(eps), _ptr(grad),
                           _stream(torch, g2.device))
    if rc != ISO_OK:
        raise IsoError(rc, "iso_soft_rank_vjp")
    return grad.reshape(g.shape)


_SoftRankFn = None


def soft_rank_fn(x, eps):
    """Differentiable soft rank: a torch.autograd.Function over soft_rank and soft_rank_vjp."""
    global _SoftRankFn
    torch = _torch()
    if _SoftRankFn is None:
        class SoftRankFn(torch.autograd.Function):
            @staticmethod
            def forward(ctx, xx, e):
                r, perm, bs = soft_rank(xx.contiguous(), e)
                ctx.save_for_backward(perm, bs)
                ctx.eps = e
                return r

            @staticmethod
            def backward(ctx, g):
                perm, bs = ctx.saved_tensors
                return soft_rank_vjp(g.contiguous(), perm, bs, ctx.eps), None

        _SoftRankFn = SoftRankFn
    return _SoftRankFn.apply(x, eps)


def vjp(g, y, w, z, block_start):
    """Backward of the fit: returns (gy, gw) (gw is None when w is None)."""
    torch = _torch()
    g2, y2, z2, b2 = _as_rows(g), _as_rows(y), _as_rows(z), _as_rows(block_start)
    code = _dtype_code(torch, y2)
    for t in (g2, z2):
        if t.shape != y2.shape or t.dtype != y2.dtype or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("g and z must match y")
    if b2.shape != y2.shape or b2.dtype != torch.uint8 or not b2.is_contiguous():
        raise ValueError("block_start must be a contiguous uint8 tensor of y's shape")
    w2 = None if w is None else _as_rows(w)
    batch, n = y2.shape
    gy = torch.empty_like(y2)
    gw = None if w2 is None else torch.empty_like(y2)
    rc = iso_vjp(_ptr(g2), _ptr(y2), _ptr(w2), _ptr(z2), _ptr(b2), _ptr(gy), _ptr(gw), batch, n, code,
                 _stream(torch, y2.device))
    if rc != ISO_OK:
        raise IsoError(rc, "iso_vjp")
    return gy.reshape(y.shape), (None if gw is None else gw.reshape(y.shape))
