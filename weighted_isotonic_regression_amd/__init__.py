"""Batched weighted L2 isotonic regression on AMD MI355X (gfx950).

The fit is computed on the GPU by hand-written HIP kernels behind a C ABI (``include/iso.h``);
this package holds those sources (``csrc/``), their build step (``build.py``), a thin ctypes
binding with the C ABI's names (``binding.py``) and the seeded input generators
(``workloads.py``).  Importing the package loads nothing; the binding loads the compiled
library on first use and raises if it is missing.
"""

__all__ = ["fit", "vjp", "iso_fit", "iso_fit_ex", "iso_vjp", "iso_workspace_bytes"]


def __getattr__(name):
    if name in __all__:
        from . import binding

        return getattr(binding, name)
    raise AttributeError(name)
