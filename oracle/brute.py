"""Exhaustive searches that pin the oracle on tiny inputs (pure Python).

TEST INFRASTRUCTURE ONLY.

* ``best_partition``: the global minimum of the k-means objective over every
  labelling of N points into at most K clusters (K^N labellings), centroids
  being the (weighted) means of the non-empty clusters.
* ``best_1d_split``: the 1D global optimum.  For scalar data an optimal
  partition consists of contiguous runs of the sorted values (the fact the
  LeanQuant "1D k-means" issue relies on when it says the 1D centroids can be
  found globally optimally), so it enumerates the C(N-1, K-1) split points.
"""
from __future__ import annotations

import itertools


def _cost(points, weights, groups):
    total = 0.0
    for members in groups:
        if not members:
            continue
        wsum = sum(weights[i] for i in members)
        d = len(points[0])
        mean = [sum(weights[i] * points[i][k] for i in members) / wsum for k in range(d)]
        for i in members:
            total += weights[i] * sum((points[i][k] - mean[k]) ** 2 for k in range(d))
    return total


def best_partition(points, K, weights=None):
    """(J*, labels*) over all K^N labellings.  points: list of d-tuples."""
    n = len(points)
    weights = weights or [1.0] * n
    best = (float("inf"), None)
    for lab in itertools.product(range(K), repeat=n):
        groups = [[i for i in range(n) if lab[i] == j] for j in range(K)]
        J = _cost(points, weights, groups)
        if J < best[0]:
            best = (J, lab)
    return best


def best_1d_split(values, K, weights=None):
    """(J*, sorted cluster means) of the optimal 1D partition into K runs."""
    n = len(values)
    weights = weights or [1.0] * n
    order = sorted(range(n), key=lambda i: values[i])
    pts = [(values[i],) for i in order]
    ws = [weights[i] for i in order]
    best = (float("inf"), None)
    for cuts in itertools.combinations(range(1, n), K - 1):
        bounds = (0,) + cuts + (n,)
        groups = [list(range(bounds[g], bounds[g + 1])) for g in range(K)]
        J = _cost(pts, ws, groups)
        if J < best[0]:
            means = [sum(ws[i] * pts[i][0] for i in g) / sum(ws[i] for i in g) for g in groups]
            best = (J, means)
    return best
