"""GPU fits of inputs with more than 2^31 elements (64-bit element offsets in every kernel).

The expected outputs follow from the definition of the fit, with no oracle run:
- a non-decreasing row is its own fit, and its canonical blocks are its runs of equal values (equal
  means pool);
- swapping the last element of one run of value k - 1 with the first of the next run, of value k,
  makes exactly those two elements one block of mean k - 1/2: the run before it ends at k - 1 <=
  k - 1/2, the run after it starts at k >= k - 1/2, and both inequalities are strict, so neither
  neighbour pools.
Runs are 512 elements long and the values stay below 2^22, so every value and every half value is an
fp32 number: the expected z is exact.  The inputs are built on the GPU piece by piece, and outputs
are compared there, so no host copy of 8 GB is made.
"""
import pytest
import torch

from weighted_isotonic_regression_amd import binding as B

pytestmark = pytest.mark.gpu

RUN = 512                      # length of a run of equal values
PIECE = 1 << 27                # elements built or compared at a time


def _runs_row(n, dev):
    """y_i = floor(i / RUN) as fp32, built piece by piece."""
    y = torch.empty(n, dtype=torch.float32, device=dev)
    for s in range(0, n, PIECE):
        e = min(n, s + PIECE)
        y[s:e] = torch.div(torch.arange(s, e, dtype=torch.int64, device=dev), RUN, rounding_mode="floor").float()
    return y


def _swap_runs_boundary(y, z_exp, p):
    """Swap elements p and p + 1 (p + 1 starts a run) in y; both become one block of mean k - 1/2."""
    a, b = float(y[p]), float(y[p + 1])
    assert b == a + 1.0
    y[p], y[p + 1] = b, a
    z_exp[p] = z_exp[p + 1] = a + 0.5


def _check_starts(bs, n, swaps, dev):
    """Block starts: every run start, except that a swapped pair starts at p, p + 1 starts nothing and
    p + 2 starts the rest of the run."""
    for s in range(0, n, PIECE):
        e = min(n, s + PIECE)
        exp = (torch.arange(s, e, dtype=torch.int64, device=dev) % RUN == 0).to(torch.uint8)
        for p in swaps:
            for q, v in ((p, 1), (p + 1, 0), (p + 2, 1)):
                if s <= q < e:
                    exp[q - s] = v
        assert torch.equal(bs[s:e], exp), "block starts differ in [%d, %d)" % (s, e)


@pytest.mark.parametrize("weighted", [False, True])
def test_row_longer_than_2_pow_31(weighted):
    """With weighted=True the unit weights are passed as an array (the weighted kernels); the
    expected fit is the same."""
    dev = torch.device("cuda:0")
    n = (1 << 31) + (1 << 20) + 37          # ragged last chunk
    print("large row: n = %d fp32, unit weights %s" % (n, "passed" if weighted else "NULL"), flush=True)
    y = _runs_row(n, dev)
    w = torch.ones(n, dtype=torch.float32, device=dev).view(1, n) if weighted else None
    z_exp = y.clone()
    # pairs at the first run boundary, across element 2^31 (also a chunk boundary), just after it,
    # and at the last whole run boundary
    last = (n // RUN) * RUN - 1
    swaps = [RUN - 1, (1 << 31) - 1, (1 << 31) + RUN - 1, last - RUN]
    for p in swaps:
        _swap_runs_boundary(y, z_exp, p)
    z = torch.empty_like(y)
    _, bs = B.fit(y.view(1, n), w, block_starts=True, out=z.view(1, n))
    bs = bs.view(n)
    torch.cuda.synchronize()
    for p in swaps:
        assert float(z[p]) == float(z_exp[p]) and float(z[p + 1]) == float(z_exp[p + 1]), p
    assert torch.equal(z, z_exp)
    _check_starts(bs, n, swaps, dev)


def test_batch_of_short_rows_past_2_pow_31():
    dev = torch.device("cuda:0")
    m = 16                                   # rows of the one-lane kernel
    rows = (1 << 27) + 3
    n = rows * m
    print("large batch: %d rows x %d fp32, unit weights" % (rows, m), flush=True)
    # row r: eight elements of value 2 (r mod 2^20), then eight of that value plus one
    y = torch.empty(n, dtype=torch.float32, device=dev)
    for s in range(0, n, PIECE):
        e = min(n, s + PIECE)
        i = torch.arange(s, e, dtype=torch.int64, device=dev)
        y[s:e] = ((i % m) // 8 + 2 * ((i // m) % (1 << 20))).float()
    z_exp = y.clone()
    # swap the run boundary (elements 7 and 8) in rows that straddle or follow element 2^31
    swap_rows = [0, (1 << 31) // m - 1, (1 << 31) // m, rows - 1]
    swaps = [r * m + 7 for r in swap_rows]
    for p in swaps:
        _swap_runs_boundary(y, z_exp, p)
    z = torch.empty_like(y)
    _, bs = B.fit(y.view(rows, m), None, block_starts=True, out=z.view(rows, m))
    bs = bs.view(n)
    torch.cuda.synchronize()
    assert torch.equal(z, z_exp)
    for s in range(0, n, PIECE):
        e = min(n, s + PIECE)
        exp = (torch.arange(s, e, dtype=torch.int64, device=dev) % 8 == 0).to(torch.uint8)
        for p in swaps:
            for q, v in ((p, 1), (p + 1, 0), (p + 2, 1)):
                if s <= q < e:
                    exp[q - s] = v
        assert torch.equal(bs[s:e], exp), "block starts differ in [%d, %d)" % (s, e)
