"""Exact rational Lloyd K-Means for tiny inputs -- TEST INFRASTRUCTURE ONLY.

Pins the fp64 oracle (``kmref.c``) on inputs small enough for exact
arithmetic with :class:`fractions.Fraction`.  Written from the definition of
Lloyd's algorithm, which the Flash-KMeans page says its kernels leave
unchanged (tech §2 opening, tech §3 "mathematical exactness"):

* assignment: squared Euclidean distance, argmin, lowest index on ties;
* update: mean of the assigned points, an empty cluster keeps its centroid;
* objective: sum of each point's distance to its assigned centroid.

Pure-Python loops; only for N*K*D up to a few thousand.
"""
from __future__ import annotations

from fractions import Fraction
from itertools import product


def _F(v):
    return v if isinstance(v, Fraction) else Fraction(v)


def sqdist(x, c):
    return sum(((_F(xj) - _F(cj)) ** 2 for xj, cj in zip(x, c)), Fraction(0))


def assign(X, C):
    """Exact argmin per point (lowest index among equal minima); returns (a, dists)."""
    a, dists = [], []
    for x in X:
        best, idx = None, 0
        for k, c in enumerate(C):
            d = sqdist(x, c)
            if best is None or d < best:
                best, idx = d, k
        a.append(idx)
        dists.append(best)
    return a, dists


def update(X, a, C_prev):
    """Exact means; an empty cluster keeps its previous centroid. Returns (C_new, counts)."""
    K, D = len(C_prev), len(C_prev[0])
    sums = [[Fraction(0)] * D for _ in range(K)]
    counts = [0] * K
    for x, k in zip(X, a):
        counts[k] += 1
        for j in range(D):
            sums[k][j] += _F(x[j])
    C_new = []
    for k in range(K):
        if counts[k] == 0:
            C_new.append([_F(v) for v in C_prev[k]])
        else:
            C_new.append([s / counts[k] for s in sums[k]])
    return C_new, counts


def objective(X, C, a):
    return sum((sqdist(x, C[k]) for x, k in zip(X, a)), Fraction(0))


def fit(X, C0, T):
    """T exact Lloyd iterations; returns (C_T, a_T, counts_T, [J_0 .. J_{T-1}])."""
    C = [[_F(v) for v in c] for c in C0]
    a, counts, J = None, [0] * len(C), []
    for _ in range(T):
        a, d = assign(X, C)
        J.append(sum(d, Fraction(0)))
        C, counts = update(X, a, C)
    return C, a, counts, J


def enumerate_min_assignment(X, C):
    """Lexicographically smallest assignment minimising sum_i d(x_i, c_{a_i}).

    Brute force over all K**N assignments.  Because the cost separates over
    points, this must equal the pointwise lowest-index argmin.
    """
    K = len(C)
    table = [[sqdist(x, c) for c in C] for x in X]
    best_cost, best_a = None, None
    for cand in product(range(K), repeat=len(X)):  # lexicographic order
        cost = sum(table[i][k] for i, k in enumerate(cand))
        if best_cost is None or cost < best_cost:
            best_cost, best_a = cost, list(cand)
    return best_a, best_cost
