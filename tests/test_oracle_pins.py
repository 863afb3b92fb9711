"""Pins of the CPU oracle against facts fixed outside of it (no GPU needed).

Each test checks the oracle against something it does not compute itself:
a library routine that is a special case (scipy's cdist + argmin, numpy's
bincount, numpy/torch IEEE conversions), a closed form, exhaustive search on
tiny inputs, or the worked example printed on the pages.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch
from scipy.spatial.distance import cdist

from oracle import brute

HERE = os.path.dirname(os.path.abspath(__file__))


def _f32_bits(a):
    return np.asarray(a, dtype=np.float32)


# ---------------------------------------------------------------- conversions

def _interesting_f32(rng, n):
    """Random float32 values plus the edge cases of the fp16/bf16 roundings."""
    u = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    vals = [u.view(np.float32)]
    vals.append(rng.standard_normal(n).astype(np.float32) * np.float32(3.0))
    vals.append((rng.standard_normal(n) * 1e-5).astype(np.float32))   # fp16 subnormals
    special = np.array([0.0, -0.0, 1.0, -1.0, 65504.0, 65519.996, 65520.0, 1e6, 6.1035156e-05,
                        5.9604645e-08, 2.9802322e-08, 2.9802326e-08, 1.0009765625, 1.00048828125,
                        1.000732421875, 1.00390625, 1.001953125, 3.4028235e38, 1.1754944e-38,
                        1e-45, np.inf, -np.inf], dtype=np.float32)
    vals.append(special)
    # exact halfway cases for fp16 and bf16 at random exponents
    m = rng.integers(0, 1 << 10, size=n).astype(np.uint32)
    e = rng.integers(100, 140, size=n).astype(np.uint32)
    halfway16 = ((e << 23) | (m << 13) | (1 << 12)).view(np.float32)
    halfway_bf = ((e << 23) | ((m & 0x7F) << 16) | (1 << 15)).view(np.float32)
    vals += [halfway16, halfway_bf]
    out = np.concatenate(vals)
    return out[np.isfinite(out) | np.isinf(out)]


def test_fp16_round_matches_numpy(orc):
    rng = np.random.default_rng(0)
    x = _interesting_f32(rng, 20000)
    x = x[~np.isnan(x)]
    got = orc.round_to(x, "f16")
    want = x.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(got, want)


def test_bf16_round_matches_torch(orc):
    rng = np.random.default_rng(1)
    x = _interesting_f32(rng, 20000)
    x = x[~np.isnan(x)]
    got = orc.round_to(x, "bf16")
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, want)


def test_decode_is_exact(orc):
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    h = allbits.view(np.float16).astype(np.float64)
    got = orc.decode(allbits, "f16")
    ok = ~np.isnan(h)
    np.testing.assert_array_equal(got[ok], h[ok])
    assert np.all(np.isnan(got[~ok]))
    b = torch.from_numpy(allbits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = orc.decode(allbits, "bf16")
    ok = ~np.isnan(b)
    np.testing.assert_array_equal(got[ok], b[ok])
    assert np.all(np.isnan(got[~ok]))


# ------------------------------------------------------------- assignment

def test_assign_matches_cdist_argmin(orc):
    rng = np.random.default_rng(2)
    B, N, d, K = 3, 300, 7, 13
    X = rng.standard_normal((B, N, d))
    Cc = rng.standard_normal((B, K, d))
    labels, d1, d2 = orc.assign(X, Cc)
    for b in range(B):
        D = cdist(X[b], Cc[b], "sqeuclidean")
        np.testing.assert_array_equal(labels[b], np.argmin(D, axis=1))
        srt = np.sort(D, axis=1)
        np.testing.assert_allclose(d1[b], srt[:, 0], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(d2[b], srt[:, 1], rtol=1e-12, atol=1e-14)


def test_assign_distance_table_exhaustive(orc):
    """Every (point, centroid) distance of a small grid, against a direct table."""
    pts = np.array(list(itertools.product([-1.0, 0.0, 0.5, 2.0], repeat=3)))  # 64 points
    cen = np.array([[0.0, 0.0, 0.0], [1.0, -1.0, 0.5], [2.0, 2.0, 2.0], [-1.0, 0.5, 0.0]])
    labels, d1, _ = orc.assign(pts[None], cen[None])
    for i, p in enumerate(pts):
        D = [float(sum((p[k] - c[k]) ** 2 for k in range(3))) for c in cen]
        assert d1[0, i] == min(D)
        assert labels[0, i] == D.index(min(D))  # list.index: first occurrence


def test_tie_goes_to_smallest_index(orc):
    X = np.array([[[0.0, 0.0], [1.0, 1.0], [5.0, 5.0]]])
    Cc = np.array([[[3.0, 3.0], [1.0, 1.0], [1.0, 1.0], [-1.0, -1.0]]])
    labels, d1, d2 = orc.assign(X, Cc)
    # point 0 is equidistant from centroids 1, 2 (d=2) and 3 (d=2)
    assert labels[0, 0] == 1 and d1[0, 0] == 2.0 and d2[0, 0] == 2.0
    assert labels[0, 1] == 1 and d1[0, 1] == 0.0 and d2[0, 1] == 0.0
    assert labels[0, 2] == 0
    nt = orc.near_tie(d1, d2)
    assert nt[0, 0] and nt[0, 1] and not nt[0, 2]


def test_near_tie_rule(orc):
    d1 = np.array([1.0, 1.0, 0.0, 0.0, 2.0])
    d2 = np.array([1.0 + 0.5e-4, 1.0 + 2e-4, 0.0, 1e-9, np.inf])
    np.testing.assert_array_equal(orc.near_tie(d1, d2), [True, False, True, False, False])


# ----------------------------------------------------------------- update

def test_update_matches_bincount(orc):
    rng = np.random.default_rng(3)
    B, N, d, K = 2, 500, 5, 11
    X = rng.standard_normal((B, N, d))
    w = rng.uniform(0.1, 1.0, size=(B, N))
    labels = rng.integers(0, K - 2, size=(B, N)).astype(np.int32)  # clusters K-2, K-1 empty
    c_old = rng.standard_normal((B, K, d)).astype(np.float32)
    for weights in (None, w):
        c_new, counts, S, W = orc.update(X, weights, labels, c_old)
        for b in range(B):
            wb = np.ones(N) if weights is None else weights[b]
            cnt = np.bincount(labels[b], minlength=K)
            Wb = np.bincount(labels[b], weights=wb, minlength=K)
            np.testing.assert_array_equal(counts[b], cnt)
            np.testing.assert_allclose(W[b], Wb, rtol=1e-13)
            for k in range(d):
                Sk = np.bincount(labels[b], weights=wb * X[b, :, k], minlength=K)
                np.testing.assert_allclose(S[b, :, k], Sk, rtol=1e-12, atol=1e-12)
                want = np.where(cnt > 0, Sk / np.where(Wb > 0, Wb, 1.0), c_old[b, :, k])
                np.testing.assert_allclose(c_new[b, :, k], want.astype(np.float32), rtol=2e-7, atol=1e-7)
            # conservation and empty clusters
            np.testing.assert_allclose(S[b].sum(axis=0), (wb[:, None] * X[b]).sum(axis=0), rtol=1e-10, atol=1e-10)
            assert counts[b].sum() == N
            np.testing.assert_array_equal(c_new[b, K - 2:], c_old[b, K - 2:])


def test_update_and_objective_from_bits_equal_the_decoded_forms(orc):
    """The bit-reading update and objective (for point sets too large to
    decode to fp64) give exactly the results of the decoded forms, which the
    closed forms above pin."""
    rng = np.random.default_rng(21)
    B, N, d, K = 3, 700, 9, 13
    for dt in ("f32", "f16", "bf16"):
        x32 = rng.standard_normal((B, N, d)).astype(np.float32)
        bits = orc.round_to(x32, dt)
        X = orc.decode(bits, dt)
        w = rng.uniform(0.1, 1.0, size=(B, N)).astype(np.float32)
        labels = rng.integers(0, K - 1, size=(B, N)).astype(np.int32)  # cluster K-1 empty
        c_old = rng.standard_normal((B, K, d)).astype(np.float32)
        Chat = orc.decode(orc.round_to(c_old, dt), dt)
        for weights in (None, w):
            want = orc.update(X, None if weights is None else weights.astype(np.float64), labels, c_old)
            got = orc.update_bits(bits, dt, weights, labels, c_old)
            for a, b_ in zip(got, want):
                np.testing.assert_array_equal(a, b_)
            Jw = orc.objective(X, None if weights is None else weights.astype(np.float64), labels, Chat)
            Jb = orc.objective_bits(bits, dt, weights, labels, Chat)
            np.testing.assert_array_equal(Jb, Jw)
    with pytest.raises(ValueError):
        orc.update_bits(bits, "bf16", None, np.full((B, N), K, np.int32), c_old)


# ------------------------------------------------------- whole iterations

def _fit_f32(orc, X32, K_init, n_iter, w=None):
    X32 = np.ascontiguousarray(X32, dtype=np.float32)
    return orc.fit(X32, "f32", w, np.ascontiguousarray(K_init, dtype=np.float32), n_iter)


def test_brute_force_tiny(orc):
    """Oracle fits never beat the exhaustive optimum and reach it from a good start."""
    rng = np.random.default_rng(4)
    for trial in range(4):
        n, K, d = 7, 3, 2
        # three separated groups (sizes 3, 2, 2) with random jitter
        centers = np.array([[0.0, 0.0], [5.0, 1.0], [1.0, 6.0]])
        grp = np.array([0, 0, 0, 1, 1, 2, 2])
        pts = (centers[grp] + 0.3 * rng.standard_normal((n, d))).astype(np.float32)
        if trial % 2:
            pts = pts[rng.permutation(n)]
        P = [tuple(float(v) for v in p) for p in pts]
        Jstar, lab_star = brute.best_partition(P, K)
        # (i) every Lloyd run from every K-subset init ends at J >= J*
        for sub in itertools.combinations(range(n), K):
            r = _fit_f32(orc, pts[None], pts[list(sub)][None], 12)
            assert r["J"][0, -1] >= Jstar - 1e-9 * max(1.0, Jstar)
        # (iii) one point of each group as init reaches the optimum exactly
        g = grp if trial % 2 == 0 else None
        if g is not None:
            init = pts[[0, 3, 5]]
            r = _fit_f32(orc, pts[None], init[None], 10)
            assert abs(r["J"][0, -1] - Jstar) <= 1e-6 * Jstar
        # (ii) the optimal means are a fixed point of one iteration
        lab_star = np.array(lab_star)
        means = np.stack([pts[lab_star == j].astype(np.float64).mean(axis=0) for j in range(K)])
        r = _fit_f32(orc, pts[None], means[None], 1)
        np.testing.assert_array_equal(r["labels"][0], lab_star)
        np.testing.assert_allclose(r["centroids"][0], means, rtol=1e-6, atol=1e-6)


def test_brute_force_weighted_tiny(orc):
    rng = np.random.default_rng(5)
    n, K = 8, 2
    pts = np.concatenate([rng.normal(0, 0.2, 4), rng.normal(3, 0.2, 4)]).astype(np.float32)[:, None]
    w = rng.uniform(0.1, 1.0, n).astype(np.float32)
    Jstar, lab = brute.best_partition([tuple(map(float, p)) for p in pts], K, [float(v) for v in w])
    r = orc.fit(pts[None], "f32", w[None], pts[[0, 4]][None], 10)
    assert abs(r["J"][0, -1] - Jstar) <= 1e-6 * Jstar
    # weighted centroid of the optimal partition
    lab = np.array(lab)
    for j in range(K):
        m = lab == j
        want = (w[m].astype(np.float64) * pts[m, 0]).sum() / w[m].astype(np.float64).sum()
        got = r["centroids"][0, r["labels"][0][m][0], 0]
        assert abs(got - want) <= 1e-6 * max(1.0, abs(want))


def test_worked_example_three_groups(orc):
    """Pages' worked example: thirteen weights in three groups, grid init."""
    g = json.load(open(os.path.join(HERE, "golden", "cache_aware_clustering_example.json")))
    v = np.array(g["weights13"], dtype=np.float32)
    K = 3
    init = np.linspace(v.astype(np.float64).min(), v.astype(np.float64).max(), K).astype(np.float32)
    r = _fit_f32(orc, v[None, :, None], init[None, :, None], 5)
    c = np.sort(r["centroids"][0, :, 0])
    printed = sorted(g["centroids13_printed"].values())
    np.testing.assert_array_equal(np.round(c.astype(np.float64), g["decimals"]), printed)
    # the partition is the three printed groups
    lab = r["labels"][0]
    for grp in g["groups13"]:
        assert len(set(lab[grp])) == 1
    assert len({lab[grp[0]] for grp in g["groups13"]}) == 3
    # and it is the global 1D optimum
    Jstar, _ = brute.best_1d_split([float(t) for t in v], K)
    assert abs(r["J"][0, -1] - Jstar) <= 1e-9
    # J is non-increasing along the fit
    assert np.all(np.diff(r["J"][0]) <= 1e-15)


def test_worked_example_two_clusters(orc):
    """Pages' worked example: the first ten weights give indices 0x5, 1x5 and two values."""
    g = json.load(open(os.path.join(HERE, "golden", "cache_aware_clustering_example.json")))
    v = np.array(g["weights10"], dtype=np.float32)
    r = _fit_f32(orc, v[None, :, None], v[None, :2, None], 10)  # first-K init
    np.testing.assert_array_equal(r["labels"][0], g["labels10_printed"])
    np.testing.assert_array_equal(np.round(r["centroids"][0, :, 0].astype(np.float64), 4),
                                  g["centroids10_printed"])
    Jstar, lab = brute.best_partition([(float(t),) for t in v], 2)
    assert abs(r["J"][0, -1] - Jstar) <= 1e-9


def test_worked_example_bad_init_is_local(orc):
    """Lloyd only reaches a local optimum: first-K init on the thirteen weights
    puts two centroids in the top group and gets stuck well above J*."""
    g = json.load(open(os.path.join(HERE, "golden", "cache_aware_clustering_example.json")))
    v = np.array(g["weights13"], dtype=np.float32)
    r = _fit_f32(orc, v[None, :, None], v[None, :3, None], 20)
    Jstar, _ = brute.best_1d_split([float(t) for t in v], 3)
    assert r["J"][0, -1] > 1e4 * Jstar
    assert abs(r["J"][0, -1] - r["J"][0, -2]) == 0.0  # a fixed point


def test_1d_global_optimum_bound(orc):
    rng = np.random.default_rng(6)
    for trial in range(6):
        n, K = 9, 3
        v = (0.02 * rng.standard_t(4, n)).astype(np.float32)
        w = rng.uniform(0.1, 1.0, n).astype(np.float32)
        Jstar, means = brute.best_1d_split([float(t) for t in v], K, [float(t) for t in w])
        init = np.linspace(float(v.min()), float(v.max()), K).astype(np.float32)
        r = orc.fit(v[None, :, None], "f32", w[None], init[None, :, None], 30)
        assert r["J"][0, -1] >= Jstar - 1e-12
    # well-separated data with grid init reaches the optimum
    v = np.concatenate([rng.normal(-1, 0.01, 3), rng.normal(0, 0.01, 3), rng.normal(1, 0.01, 3)]).astype(np.float32)
    Jstar, means = brute.best_1d_split([float(t) for t in v], 3)
    init = np.linspace(float(v.min()), float(v.max()), 3).astype(np.float32)
    r = _fit_f32(orc, v[None, :, None], init[None, :, None], 10)
    assert abs(r["J"][0, -1] - Jstar) <= 1e-9
    np.testing.assert_allclose(np.sort(r["centroids"][0, :, 0]), means, rtol=1e-6)


# ------------------------------------------------------ special cases

def test_k1_is_weighted_mean(orc):
    rng = np.random.default_rng(7)
    X = rng.standard_normal((1, 400, 6)).astype(np.float32)
    w = rng.uniform(0.1, 1, (1, 400)).astype(np.float32)
    r = orc.fit(X, "f32", w, X[:, :1], 2)
    Xd, wd = X[0].astype(np.float64), w[0].astype(np.float64)
    mean = (wd[:, None] * Xd).sum(0) / wd.sum()
    np.testing.assert_allclose(r["centroids"][0, 0], mean, rtol=1e-6, atol=1e-7)
    m32 = mean.astype(np.float32).astype(np.float64)   # the state is fp32
    J1 = (wd * ((Xd - m32) ** 2).sum(1)).sum()
    assert abs(r["J"][0, 1] - J1) <= 1e-10 * J1
    assert np.all(r["labels"] == 0) and r["counts"][0, 0] == 400
    assert np.all(np.isinf(r["d2"]))


def test_k_equals_n_identity(orc):
    rng = np.random.default_rng(8)
    X = rng.standard_normal((1, 50, 4)).astype(np.float32)
    r = orc.fit(X, "f32", None, X.copy(), 3)
    np.testing.assert_array_equal(r["labels"][0], np.arange(50))
    assert np.all(r["J"] == 0.0)
    np.testing.assert_array_equal(r["centroids"], X)
    np.testing.assert_array_equal(r["counts"][0], np.ones(50))


def test_batches_are_independent(orc):
    rng = np.random.default_rng(9)
    B, N, d, K = 4, 300, 8, 10
    X = rng.standard_normal((B, N, d)).astype(np.float16)
    bits = X.view(np.uint16)
    init = X[:, :K].astype(np.float32)
    r = orc.fit(bits, "f16", None, init, 5)
    for b in range(B):
        rb = orc.fit(bits[b:b + 1], "f16", None, init[b:b + 1], 5)
        for key in ("centroids", "labels", "counts", "J", "d1", "d2"):
            np.testing.assert_array_equal(r[key][b], rb[key][0])


def test_duplicate_centroids_and_empty_keep_old(orc):
    rng = np.random.default_rng(10)
    X = rng.standard_normal((1, 200, 3)).astype(np.float32)
    init = np.array([[[0, 0, 0], [0, 0, 0], [3, 3, 3], [50, 50, 50]]], dtype=np.float32)
    r = orc.fit(X, "f32", None, init, 1)
    assert r["counts"][0, 1] == 0 and r["counts"][0, 3] == 0
    np.testing.assert_array_equal(r["centroids"][0, 1], init[0, 1])
    np.testing.assert_array_equal(r["centroids"][0, 3], init[0, 3])
    assert set(np.unique(r["labels"][0])) <= {0, 2}


def test_lloyd_invariants_on_mixture(orc):
    """Every label is the argmin, every centroid the mean of its points, J never increases."""
    import workloads
    for dt, slack in (("f32", 1e-12), ("f16", 1e-5), ("bf16", 1e-4)):
        wl = workloads.small("gmm-b32-n65536-k1024-d128-f16", B=2, N=1500, d=12, K=24,
                             n_iter=6, dtype=dt)
        p = workloads.generate(wl)
        bits = workloads.raw_bits(p.x)
        init = p.init.numpy()
        rn = orc.fit(bits, dt, None, init, wl.n_iter)
        rp = orc.fit(bits, dt, None, init, wl.n_iter - 1)
        J = rn["J"]
        assert np.all(np.diff(J, axis=1) <= slack * J[:, :-1]), (dt, J)
        X = orc.decode(bits, dt)
        Chat = orc.decode(orc.round_to(rp["centroids"], dt), dt)
        for b in range(wl.B):
            D = cdist(X[b], Chat[b], "sqeuclidean")
            np.testing.assert_array_equal(rn["labels"][b], np.argmin(D, axis=1))
            cnt = np.bincount(rn["labels"][b], minlength=wl.K)
            for k in range(wl.d):
                s = np.bincount(rn["labels"][b], weights=X[b, :, k], minlength=wl.K)
                want = np.where(cnt > 0, s / np.maximum(cnt, 1), rp["centroids"][b, :, k])
                np.testing.assert_allclose(rn["centroids"][b, :, k], want, rtol=1e-6, atol=1e-7)


def test_fit_assigns_with_centroids_rounded_to_the_point_dtype(orc):
    """The first assignment of a fit uses the initial centroids rounded to
    the point dtype: labels and J_0 from numpy's float16 / torch's bfloat16
    rounding and scipy's cdist, with and without weights."""
    rng = np.random.default_rng(21)
    B, N, d, K = 2, 600, 5, 9
    for dt in ("f16", "bf16"):
        x32 = rng.standard_normal((B, N, d)).astype(np.float32)
        init = (rng.standard_normal((B, K, d)) * 0.7).astype(np.float32)
        w = rng.uniform(0.2, 1.0, (B, N)).astype(np.float32)
        if dt == "f16":
            bits = x32.astype(np.float16).view(np.uint16)
            X = x32.astype(np.float16).astype(np.float64)
            Chat = init.astype(np.float16).astype(np.float64)
        else:
            tb = torch.from_numpy(x32).to(torch.bfloat16)
            bits = tb.view(torch.int16).numpy().view(np.uint16)
            X = tb.double().numpy()
            Chat = torch.from_numpy(init).to(torch.bfloat16).double().numpy()
        for weights in (None, w):
            r = orc.fit(bits, dt, weights, init, 1)
            for b in range(B):
                D = cdist(X[b], Chat[b], "sqeuclidean")
                lab = np.argmin(D, axis=1)
                np.testing.assert_array_equal(r["labels"][b], lab)
                ww = np.ones(N) if weights is None else weights[b].astype(np.float64)
                J0 = (ww * D[np.arange(N), lab]).sum()
                assert abs(r["J"][b, 0] - J0) <= 1e-12 * J0, (dt, b)


def test_objective_of_labels(orc):
    """J of the assignment's labels equals the fit's J; J of other labels is larger."""
    rng = np.random.default_rng(11)
    X = rng.standard_normal((2, 300, 5)).astype(np.float32)
    w = rng.uniform(0.1, 1, (2, 300)).astype(np.float32)
    init = X[:, :7].copy()
    r = orc.fit(X, "f32", w, init, 1)
    Xd = X.astype(np.float64)
    J = orc.objective(Xd, w, r["labels"], init.astype(np.float64))
    np.testing.assert_allclose(J, r["J"][:, 0], rtol=1e-12)
    # direct formula on one batch
    lab = r["labels"][1]
    want = (w[1].astype(np.float64) * ((Xd[1] - init[1][lab].astype(np.float64)) ** 2).sum(1)).sum()
    assert abs(J[1] - want) <= 1e-10 * want
    worse = orc.objective(Xd, w, (r["labels"] + 1) % 7, init.astype(np.float64))
    assert np.all(worse > J)


# ------------------------------------------- globally optimal 1D k-means

def _groups(labels):
    """The partition of labels as a set of frozensets of point indices."""
    out = {}
    for i, l in enumerate(labels):
        out.setdefault(int(l), set()).add(i)
    return {frozenset(g) for g in out.values()}


def test_optimal_1d_matches_every_labelling(orc):
    """Exhaustive search over all K^N labellings (no contiguity assumed)."""
    rng = np.random.default_rng(21)
    for trial in range(6):
        n, K = (8, 3) if trial % 2 else (7, 2)
        v = (0.02 * rng.standard_t(4, n))
        w = rng.uniform(0.1, 1.0, n) if trial % 3 else None
        Jstar, lab = brute.best_partition([(float(t),) for t in v], K, None if w is None else list(w))
        r = orc.optimal_1d(v[None], None if w is None else w[None], K)
        assert abs(r["J"][0] - Jstar) <= 1e-12 * Jstar
        assert _groups(r["labels"][0]) == _groups(lab)
        assert r["counts"][0].sum() == n and np.all(r["counts"][0] >= 1)
        # labels are runs of the sorted values, numbered in ascending order
        assert np.all(np.diff(r["labels"][0][np.argsort(v, kind="stable")]) >= 0)


def test_optimal_1d_matches_split_enumeration(orc):
    """The C(N-1, K-1) ways to cut the sorted values into K runs."""
    rng = np.random.default_rng(22)
    for trial in range(3):
        n, K = 11, 4
        v = rng.normal(0, 1, n)
        w = rng.uniform(0.1, 1.0, n)
        Jstar, means = brute.best_1d_split(list(v), K, list(w))
        r = orc.optimal_1d(v[None], w[None], K)
        assert abs(r["J"][0] - Jstar) <= 1e-12 * Jstar
        np.testing.assert_allclose(r["means"][0], means, rtol=1e-12, atol=1e-15)


def test_optimal_1d_worked_example(orc):
    """The pages' thirteen weights: the optimum is the three printed groups
    with the printed shared values."""
    g = json.load(open(os.path.join(HERE, "golden", "cache_aware_clustering_example.json")))
    v = np.array(g["weights13"], dtype=np.float32).astype(np.float64)
    r = orc.optimal_1d(v[None], None, 3)
    assert _groups(r["labels"][0]) == {frozenset(x) for x in g["groups13"]}
    printed = sorted(g["centroids13_printed"].values())
    np.testing.assert_array_equal(np.round(r["means"][0], g["decimals"]), printed)
    Jstar, _ = brute.best_1d_split([float(t) for t in v], 3)
    assert abs(r["J"][0] - Jstar) <= 1e-12 * Jstar


def test_optimal_1d_closed_forms(orc):
    rng = np.random.default_rng(23)
    v = rng.normal(0.3, 0.1, 300)
    w = rng.uniform(0.1, 1.0, 300)
    # one run: the weighted mean and the total weighted scatter
    r = orc.optimal_1d(v[None], w[None], 1)
    m = (w * v).sum() / w.sum()
    assert abs(r["means"][0, 0] - m) <= 1e-14
    assert abs(r["J"][0] - (w * (v - m) ** 2).sum()) <= 1e-12 * r["J"][0]
    # as many runs as distinct points: every point alone, J = 0
    u = rng.permutation(np.arange(40) * 0.25 - 3.0)
    r = orc.optimal_1d(u[None], None, 40)
    assert r["J"][0] == 0.0
    np.testing.assert_array_equal(r["means"][0], np.sort(u))
    np.testing.assert_array_equal(r["labels"][0], np.argsort(np.argsort(u)))
    # a weight of 2 is the same as the point twice
    K = 5
    r1 = orc.optimal_1d(v[None], np.where(np.arange(300) == 17, 2.0, 1.0)[None], K)
    r2 = orc.optimal_1d(np.append(v, v[17])[None], None, K)
    assert abs(r1["J"][0] - r2["J"][0]) <= 1e-12 * r2["J"][0]
    np.testing.assert_allclose(r1["means"][0], r2["means"][0], rtol=1e-12)
    # translation moves the means and keeps J; scaling by 2 multiplies J by 4
    r0 = orc.optimal_1d(v[None], w[None], K)
    rt = orc.optimal_1d((v + 0.5)[None], w[None], K)
    rs = orc.optimal_1d((2.0 * v)[None], w[None], K)
    assert abs(rt["J"][0] - r0["J"][0]) <= 1e-9 * r0["J"][0]
    np.testing.assert_allclose(rt["means"][0], r0["means"][0] + 0.5, rtol=1e-12)
    assert abs(rs["J"][0] - 4 * r0["J"][0]) <= 1e-12 * r0["J"][0]


def test_optimal_1d_earliest_cut_on_ties(orc):
    """Values 2, 1, 1, 1 in three runs: J = 0 either way the equal values are
    cut; the earliest cut in sorted (value, index) order is kept."""
    r = orc.optimal_1d(np.array([[2.0, 1.0, 1.0, 1.0]]), None, 3)
    assert r["J"][0] == 0.0
    np.testing.assert_array_equal(r["labels"][0], [2, 0, 1, 1])
    np.testing.assert_array_equal(r["counts"][0], [1, 2, 1])


def test_optimal_1d_bounds_lloyd(orc):
    """Lloyd from a grid init never goes below the optimum, and the
    optimum's labels and means reproduce its J."""
    rng = np.random.default_rng(24)
    X = (0.02 * rng.standard_t(4, (3, 150))).astype(np.float32)
    w = rng.uniform(0.1, 1.0, (3, 150)).astype(np.float32)
    K = 6
    r = orc.optimal_1d(X.astype(np.float64), w.astype(np.float64), K)
    init = np.stack([np.linspace(x.min(), x.max(), K) for x in X]).astype(np.float32)[..., None]
    lloyd = orc.fit(X[..., None], "f32", w, init, 30)
    assert np.all(lloyd["J"][:, -1] >= r["J"] * (1 - 1e-12))
    Jl = orc.objective(X[..., None].astype(np.float64), w.astype(np.float64), r["labels"],
                       r["means"][..., None])
    np.testing.assert_allclose(Jl, r["J"], rtol=1e-12)


# ------------------------------------------------------------------ e-means

def _emeans(orc, X, init, batch, epochs, alpha0, floor_frac=0.1, dead_frac=0.0, eps=1e-3, u=None):
    N = X.shape[0]
    T = epochs * ((N + batch - 1) // batch)
    u = np.zeros(T * init.shape[0], np.float32) if u is None else u
    return orc.emeans(X.astype(np.float32), "f32", init.astype(np.float32), batch, epochs, alpha0, floor_frac,
                      dead_frac, eps, u)


def test_emeans_full_batch_unit_step_is_lloyd(orc):
    """One batch of all points and a constant step of 1: every update is
    S = s, N = n, i.e. Lloyd's; the last epoch's plain mean is Lloyd's last
    update.  Includes a centroid that never gets a point (kept, as in Lloyd)."""
    rng = np.random.default_rng(31)
    X = rng.normal(0, 1, (600, 5)).astype(np.float32)
    init = X[:7].copy()
    init[6] = 50.0
    for epochs in (1, 3):
        r = _emeans(orc, X, init, batch=600, epochs=epochs, alpha0=1.0, floor_frac=1.0)
        ref = orc.fit(X[None], "f32", None, init[None], epochs)
        np.testing.assert_array_equal(r["centroids"], ref["centroids"][0])
        np.testing.assert_array_equal(r["labels"], ref["labels"][0])
        np.testing.assert_array_equal(r["counts"], ref["counts"][0])
        np.testing.assert_allclose(r["J"], ref["J"][0], rtol=1e-15)


def test_emeans_single_cluster_moving_average(orc):
    """K = 1: a batch's cost is measured from the centroid before its
    update, which is the weighted mean of the batch means with weights
    a (1 - a)^age n_b (closed form, not the recursion); the cosine schedule's
    middle step is the mean of a0 and 0.1 a0."""
    rng = np.random.default_rng(32)
    X = rng.normal(0, 1, (500, 3)) * np.array([1.0, 2.0, 0.5]) + np.array([3.0, -1.0, 0.0])
    X = X.astype(np.float32)
    Xd = X.astype(np.float64)
    init = np.zeros((1, 3), np.float32)
    batch, a0 = 100, 0.4
    r = _emeans(orc, X, init, batch=batch, epochs=1, alpha0=a0, floor_frac=1.0)
    sums = [Xd[i:i + batch].sum(0) for i in range(0, 500, batch)]
    for t in range(1, 5):
        wts = [a0 * (1 - a0) ** (t - 1 - k) for k in range(t)]
        c = sum(w * s for w, s in zip(wts, sums)) / sum(w * batch for w in wts)
        c = c.astype(np.float32).astype(np.float64)   # the centroid state is float32
        J = ((Xd[t * batch:(t + 1) * batch] - c) ** 2).sum()
        assert abs(r["J"][t] - J) <= 1e-9 * J
    assert abs(r["J"][0] - (Xd[:batch] ** 2).sum()) <= 1e-9 * r["J"][0]   # from the init
    np.testing.assert_allclose(r["centroids"][0], Xd.mean(0), rtol=1e-6)   # last-epoch mean
    # cosine decay over T = 3 steps: a_1 = (a0 + 0.1 a0) / 2
    r3 = _emeans(orc, X[:300], init, batch=batch, epochs=1, alpha0=a0)
    a1 = (a0 + 0.1 * a0) / 2
    S2 = (1 - a1) * a0 * sums[0] + a1 * sums[1]
    c2 = (S2 / ((1 - a1) * a0 * batch + a1 * batch)).astype(np.float32).astype(np.float64)
    J2 = ((Xd[200:300] - c2) ** 2).sum()
    assert abs(r3["J"][2] - J2) <= 1e-9 * J2


def test_emeans_dead_cluster_splits_the_drawn_donor(orc):
    """Two tight groups and a centroid far from both: after the first batch
    it is dead; the uniform picks the donor in proportion to size (u = 0.2 the
    first group, u = 0.9 the second), the donor's points are then shared by
    the two halves of the split, and the other group is untouched."""
    rng = np.random.default_rng(33)
    A = rng.normal(0, 0.05, (200, 4)) + np.array([1.0, 1.0, 0.0, 0.0])
    Bg = rng.normal(0, 0.05, (200, 4)) + np.array([-1.0, 0.0, 2.0, 0.0])
    X = np.concatenate([A, Bg]).astype(np.float32)
    init = np.array([[1, 1, 0, 0], [-1, 0, 2, 0], [40, 40, 40, 40]], np.float32)
    for u_dead, donor, other in ((0.2, 0, 1), (0.9, 1, 0)):
        u = np.zeros(2 * 3, np.float32)
        u[2] = u_dead                     # step 0, cluster 2
        r = _emeans(orc, X, init, batch=400, epochs=2, alpha0=1.0, floor_frac=1.0, dead_frac=0.5, eps=0.05, u=u)
        grp = np.arange(400) // 200       # 0: first group, 1: second
        mine = grp == donor
        assert set(r["labels"][mine]) == {donor, 2}, "the donor's points are shared by the split pair"
        assert np.all(r["labels"][~mine] == other)
        assert r["counts"][donor] > 0 and r["counts"][2] > 0 and r["counts"][other] == 200
        np.testing.assert_allclose(r["centroids"][other], X[~mine].astype(np.float64).mean(0), rtol=1e-5)
    # no splitting without dead clusters: the far centroid keeps its place
    r = _emeans(orc, X, init, batch=400, epochs=2, alpha0=1.0, floor_frac=1.0, dead_frac=0.0)
    np.testing.assert_array_equal(r["centroids"][2], init[2])


def test_emeans_deadness_is_decided_before_the_steps_splits(orc):
    """A live cluster that a split halves below the dead line is not split
    again in the same step: which clusters are dead is fixed by the step's
    moving averages, before any split.  Scalar points: 40 at 1.9 / 2.1
    (cluster 1), 60 at 10 (cluster 2), cluster 0 far away.  After step 0
    (a = 1/2, dead below 0.45 * 100 / 3 = 15) cluster 0 is dead and draws
    cluster 1 (N = 20, halved to 10, now below the line); step 1's cost then
    follows from the split pair around cluster 1's mean, computed here from
    the definition.  Splitting cluster 1 again would move it onto cluster 2."""
    A = np.tile(np.array([1.9, 2.1], np.float32), 20)
    X = np.concatenate([A, np.full(60, 10.0, np.float32)])[:, None]
    init = np.array([[1000.0], [2.0], [10.0]], np.float32)
    u = np.zeros((2, 3), np.float32)
    u[0, 0] = 0.2    # target 0.2 * 50 = 10 lies in cluster 1's share (0, 20]
    u[0, 1] = 0.9    # used only if cluster 1 were (wrongly) split too: cluster 2
    eps = 1e-3
    r = _emeans(orc, X, init, batch=100, epochs=2, alpha0=0.5, floor_frac=0.1, dead_frac=0.45, eps=eps,
                u=u.reshape(-1))
    Ad = A.astype(np.float64)
    ck = Ad.sum() / 40.0                          # cluster 1's mean, the donor's centroid
    c0 = np.float32(ck * (1 + eps)).astype(np.float64)
    c1 = np.float32(ck * (1 - eps)).astype(np.float64)
    # step 1: the split pair takes the 40 points, cluster 2 keeps its own at distance 0
    J1 = np.minimum((Ad - c0) ** 2, (Ad - c1) ** 2).sum()
    assert abs(r["J"][1] - J1) <= 1e-9 * J1
    J0 = ((Ad - 2.0) ** 2).sum()
    assert abs(r["J"][0] - J0) <= 1e-9 * J0


def test_emeans_final_means_are_the_last_epochs_update(orc):
    rng = np.random.default_rng(34)
    X = rng.normal(0, 1, (3000, 6)).astype(np.float32)
    init = X[rng.choice(3000, 40, replace=False)].copy()
    T = 3 * 6
    r = _emeans(orc, X, init, batch=512, epochs=3, alpha0=0.3, dead_frac=0.05,
                u=rng.random(T * 40).astype(np.float32))
    c_new, counts, _, _ = orc.update(X[None].astype(np.float64), None, r["labels"][None], r["centroids"][None])
    np.testing.assert_array_equal(counts[0], r["counts"])
    live = r["counts"] > 0
    np.testing.assert_array_equal(c_new[0][live], r["centroids"][live])
    assert np.isfinite(r["J"]).all() and r["J"][-1] < r["J"][0]
