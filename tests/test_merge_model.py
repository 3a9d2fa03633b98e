"""Exact-arithmetic model of the second merge stage's rule (CPU, no GPU code):
consecutive lower hulls that share their end points are merged by bridging
every pair of neighbours, each hull keeping the vertices between its two
bridges, and a hull whose range comes out empty (or one vertex without a
strict left turn) is dropped and its new neighbours bridged, round by round.
Checked against the monotone chain on the union, with many collinear points
(integer data) and hulls of two points."""
from __future__ import annotations

from fractions import Fraction as F

import numpy as np


def cross(a, b, c):
    """> 0: b strictly below the chord from a to c."""
    return (b[0] - a[0]) * (c[1] - a[1]) - (b[1] - a[1]) * (c[0] - a[0])


def lower_hull(pts):
    h = []
    for p in pts:
        while len(h) >= 2 and cross(h[-2], h[-1], p) <= 0:
            h.pop()
        h.append(p)
    return h


def tangent(p, H, lo, hi):
    """First k in lo..hi-1 with H[k] strictly below the chord p -> H[k+1], else hi."""
    while lo < hi:
        k = (lo + hi) // 2
        if cross(p, H[k], H[k + 1]) > 0:
            hi = k
        else:
            lo = k + 1
    return lo


def bridge(L, R, adjacent):
    """(contact on L, leftmost; contact on R, rightmost) by nested bisection."""
    g, h = len(L), len(R)
    a, b, rlo = 0, g - 1, 0
    if adjacent:
        if cross(L[g - 2], L[g - 1], R[1]) > 0:
            return g - 1, 1
        b, rlo = g - 2, 1
    while a < b:
        k = (a + b) // 2
        t = tangent(L[k], R, rlo, h - 1)
        if cross(L[k], L[k + 1], R[t]) > 0:
            a = k + 1
        else:
            b = k
    return a, tangent(L[a], R, rlo, h - 1)


def merge_local(hulls):
    n = len(hulls)
    lc = [0] * n
    rc = [len(H) - 1 for H in hulls]
    for g in range(n - 1):
        rc[g], lc[g + 1] = bridge(hulls[g], hulls[g + 1], True)
    alive = list(range(n))
    while True:
        drop = []
        for t in range(1, len(alive) - 1):
            p, h, q = alive[t - 1], alive[t], alive[t + 1]
            c, d = lc[h], rc[h]
            if c > d or (c == d and not cross(hulls[p][rc[p]], hulls[h][c], hulls[q][lc[q]]) > 0):
                drop.append(h)
        if not drop:
            break
        alive = [h for h in alive if h not in drop]
        for t in range(len(alive) - 1):
            g, h = alive[t], alive[t + 1]
            if h > g + 1:
                rc[g], lc[h] = bridge(hulls[g], hulls[h], False)
    return [v for h in alive for v in hulls[h][lc[h]:rc[h] + 1]]


def test_local_bridge_merge_is_the_hull_of_the_union():
    rng = np.random.default_rng(2024)
    for case in range(400):
        n = int(rng.integers(2, 160))
        run = int(rng.integers(1, 24))
        kind = case % 3
        if kind == 0:
            y = rng.integers(-3, 4, n)
        elif kind == 1:
            y = np.sort(rng.integers(0, 6, n))[::-1] + rng.integers(-1, 2, n)
        else:
            y = rng.integers(-50, 50, n) + np.arange(n) // 3
        S = np.concatenate([[0], np.cumsum(y)])
        pts = [(F(i), F(int(S[i]))) for i in range(n + 1)]
        hulls = [lower_hull(pts[c:min(n, c + run) + 1]) for c in range(0, n, run)]
        assert merge_local(hulls) == lower_hull(pts), (case, n, run)
