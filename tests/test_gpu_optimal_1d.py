"""GPU parity of the globally optimal 1D k-means against the oracle.

The optimum J* is unique; the partition that reaches it need not be (equal
values, or two cuts whose costs agree to rounding).  So J is compared to
float64 rounding (both sides compute in float64: relative 1e-9, plus 1e-12
of the row's total weighted square for the prefix sums), and the
partition is compared exactly where it agrees with the oracle's; where it
does not, it must be valid: runs of the sorted (value, index) order, the
stated counts, centroids that are the runs' weighted means, and the oracle's
cost of the GPU's own partition equal to J*.  Full-size rows are checked on a
sample of rows against the oracle and on every row through properties
(runs, counts, J not above the GPU's own Lloyd fit).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import parity

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def km():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_lloyd_means_03_amd as km
    km.load()
    return km


def _check_runs(x, labels, counts, K, what):
    """Labels are runs 0..K-1 of the rows sorted by (value, index), with the counts given."""
    B, N = x.shape
    order = np.lexsort((np.broadcast_to(np.arange(N), (B, N)), x), axis=-1)
    ls = np.take_along_axis(labels, order, axis=-1)
    assert ls.min() >= 0 and ls.max() < K, what
    assert np.all(np.diff(ls, axis=-1) >= 0), f"{what}: labels are not runs of the sorted values"
    got = np.stack([np.bincount(l, minlength=K) for l in labels])
    np.testing.assert_array_equal(got, counts, err_msg=what)
    assert np.all(counts >= 1), f"{what}: an empty run"


def _compare(km, x, w, K, what, rows=None):
    """GPU optimum of x [B,N] (torch, CPU) against the oracle on the given rows."""
    xd = x.cuda()
    wd = None if w is None else w.cuda()
    cen, lab, cnt, J = km.kmeans_optimal_1d(xd, K, weights=wd)
    torch.cuda.synchronize()
    cen, lab, cnt, J = cen.cpu().numpy(), lab.cpu().numpy(), cnt.cpu().numpy(), J.cpu().numpy()
    X = oracle.decode(workloads.raw_bits(x), workloads.dtype_name(x))
    _check_runs(X, lab, cnt, K, what)
    rows = np.arange(x.shape[0]) if rows is None else rows
    Xr = X[rows]
    wr = None if w is None else w.numpy()[rows].astype(np.float64)
    ref = oracle.optimal_1d(Xr, wr, K)
    # the GPU costs runs from float64 prefix sums of w*x^2, whose absolute
    # rounding is at most about N * 2^-53 of their total (below 1e-12 of it for
    # N <= 4096); J* itself is compared at 1e-9 relative
    scale = ((1.0 if wr is None else wr) * Xr * Xr).sum(-1)
    tol = 1e-9 * np.abs(ref["J"]) + 1e-12 * scale
    assert np.all(np.abs(J[rows] - ref["J"]) <= tol), f"{what}: J {J[rows]} vs {ref['J']}"
    for t, b in enumerate(rows):
        if np.array_equal(lab[b], ref["labels"][t]):
            np.testing.assert_array_equal(cnt[b], ref["counts"][t])
        else:
            # another partition: it must reach J* itself
            means = np.array([np.average(Xr[t][lab[b] == c], weights=None if wr is None else wr[t][lab[b] == c])
                              for c in range(K)])
            Jg = oracle.objective(Xr[t][None, :, None], None if wr is None else wr[t][None], lab[b][None],
                                  means[None, :, None])[0]
            assert abs(Jg - ref["J"][t]) <= tol[t], f"{what} row {b}: GPU partition costs {Jg}, J* {ref['J'][t]}"
        # centroids: the weighted means of the GPU's runs
        W = np.ones_like(Xr[t]) if wr is None else wr[t]
        want = np.array([(W * Xr[t])[lab[b] == c].sum() / W[lab[b] == c].sum() for c in range(K)])
        parity.check_centroids(cen[b][:, None], want[:, None], what)
        assert np.all(np.diff(cen[b]) >= 0), f"{what}: centroids not ascending"
    return cen, lab, cnt, J


def _rows(B, N, dtype, seed, weighted=True):
    rng = np.random.default_rng(seed)
    x = torch.from_numpy((0.02 * rng.standard_t(4.0, size=(B, N))).astype(np.float32)).to(DT[dtype])
    w = torch.from_numpy(rng.uniform(0.1, 1.0, (B, N)).astype(np.float32)) if weighted else None
    return x, w


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("B,N,K,weighted", [
    (6, 1000, 16, True), (4, 1000, 8, False), (3, 777, 5, True), (5, 64, 1, True),
    (4, 300, 64, True), (2, 4096, 16, True), (3, 2049, 3, False), (8, 2, 2, True), (8, 1, 1, False),
    (2, 40, 40, True),
])
def test_optimal_parity(km, dtype, B, N, K, weighted):
    x, w = _rows(B, N, dtype, seed=B * 7 + N + K, weighted=weighted)
    _compare(km, x, w, K, f"optimal {dtype} B{B} N{N} K{K} w{weighted}")


def test_optimal_duplicates_and_constant_rows(km):
    rng = np.random.default_rng(3)
    # few distinct values, each many times; K above and below their number
    v = np.repeat(rng.normal(0, 1, 12), 9)[rng.permutation(108)].astype(np.float32)
    x = torch.from_numpy(np.stack([v, v[::-1].copy(), np.full(108, 0.25, np.float32)]))
    w = torch.from_numpy(rng.uniform(0.1, 1.0, (3, 108)).astype(np.float32))
    for K in (5, 12, 20):
        _compare(km, x, w, K, f"duplicates K{K}")
        _compare(km, x, None, K, f"duplicates unweighted K{K}")


def test_optimal_worked_example(km):
    """The pages' thirteen weights: the three printed groups and values."""
    g = json.load(open(os.path.join(HERE, "golden", "cache_aware_clustering_example.json")))
    x = torch.tensor([g["weights13"]], dtype=torch.float32)
    cen, lab, cnt, J = _compare(km, x, None, 3, "worked example")
    groups = {frozenset(np.where(lab[0] == c)[0].tolist()) for c in range(3)}
    assert groups == {frozenset(t) for t in g["groups13"]}
    np.testing.assert_array_equal(np.round(cen[0].astype(np.float64), g["decimals"]),
                                  sorted(g["centroids13_printed"].values()))


def test_optimal_full_rows(km):
    """The 4096 x 4096 weighted rows at K = 16: sampled rows against the
    oracle, every row through the run structure and J* <= the GPU's Lloyd J."""
    wl = workloads.WORKLOADS["rows1d-b4096-n4096-k16-f32"]
    p = workloads.generate(wl)
    x, w = p.x[..., 0], p.w
    rows = np.array([0, 1, 777, 2048, 4095])
    cen, lab, cnt, J = _compare(km, x, w, 16, "full rows", rows=rows)
    _, _, _, Jl = km.kmeans_fit(p.x.cuda(), p.init.cuda(), wl.n_iter, weights=w.cuda())
    torch.cuda.synchronize()
    Jl = Jl.cpu().numpy()[:, -1]
    assert np.all(J <= Jl * (1 + 1e-9)), "the optimum is above a Lloyd fit"
    assert np.mean(J < Jl * (1 - 1e-6)) > 0.5  # and strictly better on most rows


def test_optimal_rejects(km):
    x = torch.zeros(2, 10, device="cuda")
    with pytest.raises(km.KMeansError, match="K <= N"):
        km.kmeans_optimal_1d(x, 11)
    with pytest.raises(km.KMeansError, match="N <= 4096"):
        km.kmeans_optimal_1d(torch.zeros(1, 4097, device="cuda"), 4)
