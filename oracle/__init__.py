"""TEST INFRASTRUCTURE ONLY: the CPU oracle for batched weighted L2 isotonic regression.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg may import
this package.  The GPU library never imports, links or calls it, and it shares no code with
the GPU path.

Contents
--------
``pav``            the plain C pool-adjacent-violators scan in fp64 (``iso_oracle.c``).
``vjp``            the block-averaging backward over given block starts (``iso_oracle.c``).
``exact``          exact-rational characterisations used to pin ``pav``: the max-min
                   block-average formula, the explicit lower convex hull of the cumulative
                   sum diagram, and the KKT certificate.
``softrank``       the soft rank (projection onto the permutahedron) and its backward, built
                   on ``pav`` and ``vjp``.
"""
from .native import build, pav, vjp, ORACLE_FLAG_NONFINITE, ORACLE_FLAG_WEIGHT  # noqa: F401
from . import exact  # noqa: F401
from . import softrank  # noqa: F401
