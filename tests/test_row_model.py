"""Models, in plain Python, of two design rules of the one-row-per-workgroup kernel (k_row in
csrc/iso_row.h), checked on the CPU.

1. The merge procedure, in exact rational arithmetic.  Leaves of four points decide each inner
   point by testing it against every pair of points around it.  Neighbouring hulls are merged
   level by level by their bridge, found three ways:
   - a concatenation when the union is convex at the shared point s;
   - the candidate search: for each vertex a of the left hull, bisect the right hull for the
     tangent point b(a), then keep a if its predecessor lies strictly above the line a b(a) and
     its successor on or above it;
   - the pair test: (alpha, beta) is the bridge iff alpha's predecessor is strictly above the line
     alpha beta, its successor on or above, beta's successor strictly above and its predecessor
     on or above.
   With exact turns exactly one candidate and exactly one pair must pass, and the final hull must
   equal a direct monotone-chain hull of the whole diagram ("Merge Hulls Without Copying
   Vertices: GPU Isotonic Regression", Section 2 and Section 3.2, Lemma 4.2).

2. LDS ownership under wavefront-only syncs.  At level r a merge of nodes 2j and 2j + 1 is done
   by threads j 2^(r+1) .. (j + 1) 2^(r+1) - 1.  Node k's vertex count sits at index k 2^r, its
   list at offset k m, and its bridge slots at index j 2^(r+1).  Every word a level touches must
   then have been touched last by threads of the same group, so that levels whose groups fit in
   one wavefront only need that wavefront to sync.  The check also shows that indexing counts by
   node number would break the rule.

Nothing here runs on the GPU or reads the kernel; these are the rules the kernel was written to.
"""
from fractions import Fraction as F
import random

import pytest


def turn(P, i, j, k):
    (ax, ay), (bx, by), (cx, cy) = P[i], P[j], P[k]
    return (bx - ax) * (cy - ay) - (by - ay) * (cx - ax)


def left(P, i, j, k):
    return turn(P, i, j, k) > 0


def chain_hull(P, lo, hi):
    """Lower hull of points lo..hi by the monotone chain, collinear middle points dropped."""
    st = []
    for k in range(lo, hi + 1):
        while len(st) >= 2 and not left(P, st[-2], st[-1], k):
            st.pop()
        st.append(k)
    return st


def model_hull(P, n, stats):
    """The kernel's procedure: leaves of four points, then merge levels.  Lists hold a node's
    vertices without its end point.  Returns the root hull's vertices, end point included."""
    nodes = (n + 3) // 4
    L = []
    for t in range(nodes):
        e0 = 4 * t
        c = min(4, n - e0)
        vt = [k < c for k in range(4)]
        for k in range(1, 4):
            for a in range(k):
                for b in range(k + 1, 5):
                    if b <= c and vt[k] and not left(P, e0 + a, e0 + k, e0 + b):
                        vt[k] = False
        L.append([e0 + k for k in range(4) if vt[k]])
    m = 4
    while nodes > 1:
        merges = nodes // 2
        nxt = []
        for j in range(merges):
            LA, LB = L[2 * j], L[2 * j + 1]
            cA, cB = len(LA), len(LB)
            s, e = (2 * j + 1) * m, min((2 * j + 2) * m, n)
            assert LB[0] == s

            def Ai(i):
                return LA[i] if i < cA else s

            def Bk(k):
                return LB[k] if k < cB else e

            b1 = LB[1] if cB > 1 else e
            if left(P, LA[cA - 1], s, b1):
                bridge = (cA, 1)
                stats["convex"] += 1
            else:
                cands = []
                for i in range(cA + 1):
                    a = Ai(i)
                    lo, hi = 1, cB
                    while lo < hi:
                        mid = (lo + hi) // 2
                        if left(P, a, Bk(mid), Bk(mid + 1)):
                            hi = mid
                        else:
                            lo = mid + 1
                    b = Bk(lo)
                    ok = (i == 0 or left(P, Ai(i - 1), a, b)) and (i == cA or not left(P, a, Ai(i + 1), b))
                    if ok:
                        cands.append((i, lo))
                pairs = []
                for i in range(cA + 1):
                    for k in range(1, cB + 1):
                        a, b = Ai(i), Bk(k)
                        ok = ((i == 0 or left(P, Ai(i - 1), a, b)) and (i == cA or not left(P, a, Ai(i + 1), b))
                              and (k == cB or left(P, a, b, Bk(k + 1))) and (k == 1 or not left(P, a, Bk(k - 1), b)))
                        if ok:
                            pairs.append((i, k))
                assert len(cands) == 1, cands
                assert pairs == cands, (pairs, cands)
                bridge = cands[0]
                stats["searched"] += 1
            al, be = bridge
            nxt.append([Ai(k) for k in range(al + 1)] + LB[be:cB])
        if nodes & 1:
            nxt.append(L[nodes - 1])
        L = nxt
        nodes = (nodes + 1) // 2
        m *= 2
    return L[0] + [n]


def diagram(y, w):
    P = [(F(0), F(0))]
    for yi, wi in zip(y, w):
        P.append((P[-1][0] + wi, P[-1][1] + wi * F(yi)))
    return P


def rows(seed, count):
    rng = random.Random(seed)
    for trial in range(count):
        n = rng.choice([17, 18, 31, 64, 100, 257, 700]) if trial % 5 else rng.randint(17, 300)
        kind = trial % 6
        if kind == 0:
            y = [rng.gauss(0, 1) for _ in range(n)]
        elif kind == 1:
            y = [i / n + rng.gauss(0, 0.3) for i in range(n)]
        elif kind == 2:
            y = [float(rng.randint(0, 3)) for _ in range(n)]
        elif kind == 3:
            y = [1.5] * n
        elif kind == 4:
            y = [float(-i) for i in range(n)]
        else:
            y = [float(i * i) for i in range(n)]
        w = [F(rng.randint(1, 4)) for _ in range(n)] if trial % 2 else [F(1)] * n
        yield n, y, w


def test_merge_procedure_matches_direct_hull():
    stats = {"convex": 0, "searched": 0}
    for n, y, w in rows(7, 120):
        P = diagram(y, w)
        assert model_hull(P, n, stats) == chain_hull(P, 0, n)
    assert stats["convex"] > 100 and stats["searched"] > 100, stats


def test_leaf_rule_on_collinear_and_convex_points():
    # four collinear increments: only the leaf's first point is a vertex before its end
    P = diagram([2.0] * 4, [F(1)] * 4)
    assert model_hull(P, 4, {"convex": 0, "searched": 0}) == [0, 4]
    # strictly convex diagram: every point is a vertex
    P = diagram([1.0, 2.0, 3.0, 4.0, 5.0, 6.0, 7.0, 8.0], [F(1)] * 8)
    assert model_hull(P, 8, {"convex": 0, "searched": 0}) == list(range(9))


def ownership_violations(n, count_index):
    """Walks the levels recording, for every LDS word, the thread range that touched it last;
    returns the accesses made after a wavefront-only sync by a group that does not contain that
    range."""
    nodes = (n + 3) // 4
    last, bad = {}, []

    def touch(key, lo, hi, wave_only):
        if key in last and wave_only:
            plo, phi = last[key]
            if not (lo <= plo and phi <= hi):
                bad.append((key, (plo, phi), (lo, hi)))
        last[key] = (lo, hi)

    for t in range(nodes):
        touch(("C", 0, count_index(t, 0)), t, t + 1, False)
        for k in range(4):
            touch(("L", 0, 4 * t + k), t, t + 1, False)
    m, cur, r, wave_only = 4, 0, 0, True  # the leaves end with a wavefront sync
    while nodes > 1:
        merges, tpm = nodes // 2, 2 << r
        for j in range(merges + (nodes & 1)):
            lo, hi = j * tpm, (j + 1) * tpm
            kids = (2 * j, 2 * j + 1) if j < merges else (nodes - 1,)
            for kid in kids:
                touch(("C", cur, count_index(kid, r)), lo, hi, wave_only)
                for k in range(m):
                    touch(("L", cur, kid * m + k), lo, hi, wave_only)
                    touch(("L", cur ^ 1, kid * m + k), lo, hi, wave_only)
            touch(("C", cur ^ 1, count_index(j, r + 1)), lo, hi, wave_only)
            if j < merges:
                touch(("S", j * tpm), lo, hi, wave_only)
        nodes, m, cur, r = (nodes + 1) // 2, 2 * m, cur ^ 1, r + 1
        wave_only = (2 * tpm <= 64) and nodes > 1
        if not wave_only:
            last.clear()  # a workgroup barrier orders everything before it
    return bad


@pytest.mark.parametrize("n", [17, 64, 100, 257, 999, 2048, 2049, 3001, 4095, 4096])
def test_lds_ownership_with_first_leaf_indexing(n):
    assert ownership_violations(n, lambda k, r: k << r) == []


def test_node_number_indexing_would_race():
    assert ownership_violations(100, lambda k, r: k)
