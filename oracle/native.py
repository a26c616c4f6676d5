"""TEST INFRASTRUCTURE ONLY: ctypes wrapper and gcc build of the C oracle ``iso_oracle.c``.

The C file is compiled with plain ``gcc -O2`` (no fast-math, no FMA contraction) into
``oracle/_build/libiso_oracle.so``.  The wrapper converts inputs to contiguous fp64 numpy
arrays and returns fp64 results.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

ORACLE_FLAG_NONFINITE = 1
ORACLE_FLAG_WEIGHT = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "iso_oracle.c")
_OUT_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_OUT_DIR, "libiso_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc.  Returns the path of the shared library."""
    os.makedirs(_OUT_DIR, exist_ok=True)
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            lib.iso_oracle_fit.argtypes = [P, P, P, P, P, ctypes.c_int64, ctypes.c_int64]
            lib.iso_oracle_fit.restype = ctypes.c_int
            lib.iso_oracle_fit_dir.argtypes = [P, P, P, P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
            lib.iso_oracle_fit_dir.restype = ctypes.c_int
            lib.iso_oracle_vjp.argtypes = [P, P, P, P, P, P, P, ctypes.c_int64, ctypes.c_int64]
            lib.iso_oracle_vjp.restype = ctypes.c_int
            _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _as2d(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if a.ndim == 1:
        a = a[None, :]
    if a.ndim != 2:
        raise ValueError("expected a 1-D row or a 2-D [batch, n] array")
    return a


def pav(y, w=None, *, return_blocks: bool = False, decreasing: bool = False):
    """Fit every row of ``y`` (1-D or [batch, n]) with weights ``w`` (same shape or None);
    ``decreasing=True`` fits z_0 >= ... >= z_{n-1} instead.

    Returns ``z`` (fp64, same shape as ``y``), and with ``return_blocks=True`` also the
    block-start mask (uint8, same shape) and the per-row flags (uint32, [batch]).
    """
    y_in = np.asarray(y)
    y2 = _as2d(y_in)
    w2 = None if w is None else _as2d(w)
    if w2 is not None and w2.shape != y2.shape:
        raise ValueError("w must have the shape of y")
    batch, n = y2.shape
    z = np.empty_like(y2)
    bs = np.empty(y2.shape, dtype=np.uint8)
    flags = np.empty(batch, dtype=np.uint32)
    rc = _load().iso_oracle_fit_dir(_ptr(y2), _ptr(w2), _ptr(z), _ptr(bs), _ptr(flags), batch, n,
                                    1 if decreasing else 0)
    if rc != 0:
        raise RuntimeError("iso_oracle_fit failed with code %d" % rc)
    if y_in.ndim == 1:
        z, bs = z[0], bs[0]
    if return_blocks:
        return z, bs, flags
    return z


def vjp(g, y, w, z, block_start):
    """Backward of the fit over the given blocks.  Returns (gy, gw); gw is None when w is None."""
    y_in = np.asarray(y)
    g2, y2, z2 = _as2d(g), _as2d(y), _as2d(z)
    w2 = None if w is None else _as2d(w)
    b2 = np.ascontiguousarray(np.asarray(block_start, dtype=np.uint8))
    if b2.ndim == 1:
        b2 = b2[None, :]
    batch, n = y2.shape
    gy = np.empty_like(y2)
    gw = None if w2 is None else np.empty_like(y2)
    rc = _load().iso_oracle_vjp(_ptr(g2), _ptr(y2), _ptr(w2), _ptr(z2), _ptr(b2), _ptr(gy), _ptr(gw),
                                batch, n)
    if rc != 0:
        raise RuntimeError("iso_oracle_vjp failed with code %d" % rc)
    if y_in.ndim == 1:
        gy = gy[0]
        gw = None if gw is None else gw[0]
    return gy, gw
