"""GPU parity of e-means (kmeans_emeans) against the oracle.

e-means is a trajectory: every step's assignment depends on every earlier
step.  Where the points sit far from every decision boundary (well
separated mixtures, init inside the components) both sides take the same
labels at every step, and the whole run is compared: the last epoch's labels
and counts exactly, each step's objective at 1e-3 relative (the GPU's fp32
expanded-form distances), centroids at the Lloyd tolerance.  A split puts
two centroids inside one component, which makes near ties in later steps,
so splits are checked exactly on one-step runs (the resurrected centroids
are visible there: the last-epoch mean leaves clusters without points
alone), including chains of splits from one donor across several LDS
windows, and a cluster that draws itself.
Longer runs with splits are checked through what holds on any trajectory:
the counts are the label histogram, every cluster with points sits at the
plain mean of its last-epoch points, the first step's objective equals the
oracle's, and the final cost is close to the oracle's.  A full-batch run
with unit steps is Lloyd, checked against kmeans_fit.  The full-size
workload is checked on sampled labels of its first batch and on the same
properties.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import parity

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def km():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_lloyd_means_03_amd as km
    km.load()
    return km


def _separated(N, d, K, dtype, seed, scale=3.0, sigma=0.1):
    """K well separated components (means scale * N(0, 1), std sigma), the
    points in random order; init is one point of every component."""
    rng = np.random.default_rng(seed)
    if d == 1:
        means = (np.arange(K) * scale + rng.uniform(0, 0.1 * scale, K))[:, None]
    else:
        means = scale * rng.standard_normal((K, d))
    comp = rng.permutation(np.arange(N) % K)
    x32 = (means[comp] + sigma * rng.standard_normal((N, d))).astype(np.float32)
    x = torch.from_numpy(x32).to(DT[dtype])
    first = np.array([np.flatnonzero(comp == k)[0] for k in range(K)])
    init = x[torch.from_numpy(first)].float()
    return x, init


def _run(km, x, init, batch, epochs, alpha0, floor, dead_frac, eps, u):
    ud = None if u is None else torch.from_numpy(u).cuda()
    cen, lab, cnt, J = km.kmeans_emeans(x.cuda(), init.cuda(), batch, epochs, alpha0, floor, dead_frac, eps,
                                        uniforms=ud, labels=True)
    torch.cuda.synchronize()
    return cen.cpu().numpy(), lab.cpu().numpy(), cnt.cpu().numpy(), J.cpu().numpy()


def _oracle(x, init, batch, epochs, alpha0, floor, dead_frac, eps, u):
    N = x.shape[0]
    K = init.shape[0]
    T = epochs * ((N + batch - 1) // batch)
    uu = np.zeros((T, K), np.float32) if u is None else u
    return oracle.emeans(workloads.raw_bits(x), workloads.dtype_name(x), init.numpy(), batch, epochs, alpha0,
                         floor, dead_frac, eps, uu)


@pytest.mark.parametrize("dtype,N,d,K,batch,epochs", [
    ("f16", 10000, 32, 40, 2500, 3),
    ("bf16", 9001, 64, 100, 2048, 2),    # ragged last batch
    ("f32", 6000, 33, 24, 1000, 2),      # padded rows
    ("f16", 12000, 128, 256, 4096, 2),   # several centroid tiles
    ("f32", 5000, 1, 12, 1200, 3),       # scalar points: the bracketing assignment
    ("f16", 4001, 1, 5, 1001, 2),        # scalar points, K <= 16, batches not 4-aligned
    ("bf16", 3000, 7, 10, 5000, 2),      # batch above N: one full batch per epoch
    ("bf16", 8000, 96, 200, 2048, 2),    # 96-wide rows
    ("f16", 8192, 32, 4096, 2048, 1),    # 4 point groups, 16 tiles: centroid slices
])
def test_emeans_trajectory_parity(km, dtype, N, d, K, batch, epochs):
    what = f"emeans {dtype} N{N} d{d} K{K} batch{batch}"
    x, init = _separated(N, d, K, dtype, seed=N + d + K)
    got = _run(km, x, init, batch, epochs, 0.6, 0.1, 0.0, 0.0, None)
    ref = _oracle(x, init, batch, epochs, 0.6, 0.1, 0.0, 0.0, None)
    cen, lab, cnt, J = got
    np.testing.assert_array_equal(lab, ref["labels"], err_msg=what)
    np.testing.assert_array_equal(cnt, ref["counts"], err_msg=what)
    np.testing.assert_allclose(J, ref["J"], rtol=1e-3, err_msg=what)
    parity.check_centroids(cen[None], ref["centroids"][None], what)


def test_emeans_short_last_batch_with_more_groups(km):
    """A last batch just short of the full one can be assigned in more point
    groups than the full batch (one column block per wave when its groups
    would not fill the chip): 131072 points make 256 groups of 512, 130000
    make 508 groups of 256.  Every group's objective partial must fit the
    workspace; the labels stay in the workspace here, next to the partials."""
    N, d, K, batch = 131072 + 130000, 16, 64, 131072
    x, init = _separated(N, d, K, "f16", seed=77)
    T = 2
    cen, _, cnt, J = km.kmeans_emeans(x.cuda(), init.cuda(), batch, 1, 0.6, 0.1, 0.0, 0.0)
    torch.cuda.synchronize()
    ref = _oracle(x, init, batch, 1, 0.6, 0.1, 0.0, 0.0, None)
    np.testing.assert_array_equal(cnt.cpu().numpy(), ref["counts"])
    np.testing.assert_allclose(J.cpu().numpy(), ref["J"], rtol=1e-3)
    parity.check_centroids(cen.cpu().numpy()[None], ref["centroids"][None], "short last batch")
    assert J.numel() == T


def test_emeans_full_batch_unit_steps_is_lloyd(km):
    """batch >= N, alpha = 1 at every step, no splits: each step is one Lloyd
    iteration, so the run is kmeans_fit with n_iter = epochs."""
    wl = workloads.small("gmm-n1m-k8192-d128-f16", N=20000, K=128, n_iter=4, seed=11)
    p = workloads.generate(wl)
    x = p.x[0]
    cen, lab, cnt, J = _run(km, x, p.init[0], 1 << 20, 4, 1.0, 1.0, 0.0, 0.0, None)
    cf, lf, nf, Jf = km.kmeans_fit(p.x.cuda(), p.init.cuda(), 4)
    torch.cuda.synchronize()
    lf, Jf = lf[0].cpu().numpy(), Jf[0].cpu().numpy()
    np.testing.assert_allclose(J, Jf, rtol=1e-6)
    assert np.mean(lab != lf) <= 1e-3
    if np.array_equal(lab, lf):
        np.testing.assert_array_equal(cnt, nf[0].cpu().numpy())
        parity.check_centroids(cen[None], cf.cpu().numpy(), "unit steps vs kmeans_fit")


def _split_case(K, live, N, d, dtype, seed, small=None):
    """`live` separated components hold the points; the other K - live
    centroids start far away and receive none.  `small`: (cluster, points)
    gives one live component only that many points."""
    rng = np.random.default_rng(seed)
    means = 3.0 * rng.standard_normal((live, d))
    comp = np.arange(N) % live
    if small is not None:
        c, n = small
        idx = np.flatnonzero(comp == c)
        comp[idx[n:]] = (c + 1) % live
    comp = rng.permutation(comp)
    x32 = (means[comp] + 0.1 * rng.standard_normal((N, d))).astype(np.float32)
    x = torch.from_numpy(x32).to(DT[dtype])
    # live centroids at scattered cluster indices, the rest far out
    order = rng.permutation(K)
    live_idx = np.sort(order[:live])
    init = np.empty((K, d), np.float32)
    init[:] = (1000.0 + np.arange(K)[:, None] * 10.0 + np.arange(d)[None, :]).astype(np.float32)
    for c, j in enumerate(live_idx):
        init[j] = x[int(np.flatnonzero(comp == c)[0])].float().numpy()
    return x, torch.from_numpy(init), live_idx


@pytest.mark.parametrize("dtype,K,live,d,eps", [
    ("f16", 64, 8, 32, 1e-3),
    ("bf16", 300, 5, 48, 1e-2),     # long chains: ~60 splits from every donor
    ("f32", 3000, 10, 16, 1e-3),    # three LDS windows, ~300 splits per donor
    ("f16", 1030, 1, 8, 1e-3),      # one donor halved 1029 times (its count stays a normal float64)
])
def test_emeans_split_one_step(km, dtype, K, live, d, eps):
    """One step (T = 1): the dead clusters' resurrected centroids survive the
    last-epoch mean, since they received no points."""
    N = 4000
    x, init, live_idx = _split_case(K, live, N, d, dtype, seed=K + live)
    u = workloads.emeans_uniforms(K, 1, K)
    what = f"split {dtype} K{K} live{live}"
    cen, lab, cnt, J = _run(km, x, init, N, 1, 0.5, 0.1, 0.5, eps, u)
    ref = _oracle(x, init, N, 1, 0.5, 0.1, 0.5, eps, u)
    np.testing.assert_array_equal(lab, ref["labels"], err_msg=what)
    np.testing.assert_array_equal(cnt, ref["counts"], err_msg=what)
    np.testing.assert_allclose(J, ref["J"], rtol=1e-3, err_msg=what)
    moved = ~np.all(ref["centroids"] == init.numpy(), axis=1)
    assert moved.sum() == K, f"{what}: only {moved.sum()} clusters moved"
    # float32 centroids from float64 state that differs only by the batch sums'
    # fp32 rounding on the GPU
    np.testing.assert_allclose(cen, ref["centroids"], rtol=1e-5, atol=1e-6, err_msg=what)


def test_emeans_split_skips_a_cluster_that_draws_itself(km):
    """A live cluster below the dead line can draw itself as donor: nothing
    happens to it; others draw it as a donor and halve it."""
    K, live, N, d = 40, 4, 4000, 16
    x, init, live_idx = _split_case(K, live, N, d, "f32", seed=5, small=(2, 3))
    # dead line 0.5 * N / K = 50 > the small cluster's 0.5 * 3
    ref0 = _oracle(x, init, N, 1, 0.5, 0.1, 0.5, 1e-3, np.zeros((1, K), np.float32))
    counts = ref0["counts"]
    j_small = live_idx[2]
    assert counts[j_small] == 3
    # the small cluster's own uniform lands inside its own share of the prefix
    nn = 0.5 * counts.astype(np.float64)
    P = np.concatenate([[0.0], np.cumsum(nn)])
    u = workloads.emeans_uniforms(99, 1, K)
    u[0, j_small] = np.float32((P[j_small] + 0.5 * nn[j_small]) / P[-1])
    ref = _oracle(x, init, N, 1, 0.5, 0.1, 0.5, 1e-3, u)
    cen, lab, cnt, J = _run(km, x, init, N, 1, 0.5, 0.1, 0.5, 1e-3, u)
    np.testing.assert_allclose(cen, ref["centroids"], rtol=1e-5, atol=1e-6)
    np.testing.assert_array_equal(cnt, ref["counts"])


def test_emeans_deadness_is_decided_before_the_steps_splits(km):
    """The oracle pin's case: a split halves a live cluster below the dead
    line, and it is not split again in the same step."""
    A = np.tile(np.array([1.9, 2.1], np.float32), 20)
    x = torch.from_numpy(np.concatenate([A, np.full(60, 10.0, np.float32)])[:, None])
    init = torch.tensor([[1000.0], [2.0], [10.0]])
    u = np.zeros((2, 3), np.float32)
    u[0, 0], u[0, 1] = 0.2, 0.9
    got = _run(km, x, init, 100, 2, 0.5, 0.1, 0.45, 1e-3, u)
    ref = _oracle(x, init, 100, 2, 0.5, 0.1, 0.45, 1e-3, u)
    np.testing.assert_array_equal(got[1], ref["labels"])
    # the GPU's batch sums are fp32: its centroid after step 0 is off by
    # ~1e-7 of 2.0, which moves step 1's distances of ~0.1 by ~4e-6
    # relative; a second split of cluster 1 would change J[1] by 4%
    np.testing.assert_allclose(got[3], ref["J"], rtol=1e-4)
    np.testing.assert_allclose(got[0], ref["centroids"], rtol=1e-5)


@pytest.mark.parametrize("dtype,d,K,batch,epochs,dead_frac", [
    ("f16", 32, 256, 3000, 3, 0.2),
    ("bf16", 96, 512, 4096, 2, 0.1),
    ("f32", 16, 64, 1500, 4, 0.3),
])
def test_emeans_with_splits_properties(km, dtype, d, K, batch, epochs, dead_frac):
    N = 20000
    wl = workloads.small("gmm-n1m-k8192-d128-f16", N=N, d=d, K=K, dtype=dtype, n_iter=1, seed=d + K,
                         sigma=0.15, noise_frac=0.05, ncomp=K // 2)
    p = workloads.generate(wl)
    x, init = p.x[0], p.init[0]
    T = epochs * ((N + batch - 1) // batch)
    u = workloads.emeans_uniforms(wl.seed, T, K)
    what = f"splits {dtype} d{d} K{K}"
    cen, lab, cnt, J = _run(km, x, init, batch, epochs, 0.5, 0.1, dead_frac, 1e-2, u)
    ref = _oracle(x, init, batch, epochs, 0.5, 0.1, dead_frac, 1e-2, u)
    assert lab.min() >= 0 and lab.max() < K
    np.testing.assert_array_equal(cnt, np.bincount(lab, minlength=K), err_msg=what)
    assert cnt.sum() == N
    # every cluster with last-epoch points sits at their plain mean
    X = oracle.decode(workloads.raw_bits(x)[None], dtype)
    mean_c, mean_n, _, _ = oracle.update(X, None, lab[None], cen[None])
    np.testing.assert_array_equal(mean_n[0], cnt)
    live = cnt > 0
    parity.check_centroids(cen[live][None], mean_c[0][live][None], what)
    # the first step is the same computation on both sides
    np.testing.assert_allclose(J[0], ref["J"][0], rtol=1e-3, err_msg=what)
    # and the fits end at about the same cost
    Cg = oracle.decode(oracle.round_to(cen, dtype), dtype)
    Cr = oracle.decode(oracle.round_to(ref["centroids"], dtype), dtype)
    _, dg, _ = oracle.assign(X, Cg[None])
    _, dr, _ = oracle.assign(X, Cr[None])
    assert abs(dg.sum() - dr.sum()) <= 0.05 * dr.sum(), f"{what}: final cost {dg.sum()} vs {dr.sum()}"
    # splitting keeps (almost) every cluster alive
    assert (cnt == 0).sum() <= (ref["counts"] == 0).sum() + K // 50


def test_emeans_empty_and_rejects(km):
    init = torch.randn(8, 16, device="cuda")
    cen, lab, cnt, J = km.kmeans_emeans(torch.zeros(0, 16, device="cuda", dtype=torch.float16), init, 100, 2, 0.5)
    torch.cuda.synchronize()
    assert torch.equal(cen, init) and J.numel() == 0 and int(cnt.abs().sum()) == 0
    x = torch.zeros(100, 16, device="cuda", dtype=torch.float16)
    with pytest.raises(km.KMeansError, match="uniforms"):
        km.kmeans_emeans(x, init, 10, 1, 0.5, dead_frac=0.5)
    with pytest.raises(km.KMeansError, match="alpha0"):
        km.kmeans_emeans(x, init, 10, 1, 0.0)


def test_emeans_full_workload(km):
    """The measured workload: one epoch at full size.  Sampled points of the
    first batch (assigned against init) against the oracle, then the
    properties of the last epoch."""
    wl = workloads.WORKLOADS["emeans-n1m-k16384-d96-bf16"]
    p = workloads.generate(wl)
    x, init = p.x[0], p.init[0]
    N, K, batch = wl.N, wl.K, wl.em_batch
    T = (N + batch - 1) // batch
    u = workloads.emeans_uniforms(wl.seed, T, K)
    cen, lab, cnt, J = _run(km, x, init, batch, 1, wl.em_alpha0, wl.em_floor, wl.em_dead_frac, wl.em_eps, u)
    rows = np.random.default_rng(0).choice(batch, size=1500, replace=False)
    xb = workloads.raw_bits(x)[rows][None]
    _, _, ref_lab, d1, d2 = parity.oracle_assign(xb, wl.dtype, init.numpy()[None])
    parity.check_labels(lab[rows][None], ref_lab, d1, d2, "first batch")
    np.testing.assert_array_equal(cnt, np.bincount(lab, minlength=K))
    assert np.all(np.isfinite(J)) and np.all(J > 0)
    # clusters with points sit at the plain mean of their points (sampled clusters)
    sel = np.random.default_rng(1).choice(np.flatnonzero(cnt > 0), size=64, replace=False)
    X = oracle.decode(workloads.raw_bits(x), wl.dtype)
    for j in sel:
        m = X[lab == j].mean(0)
        assert np.linalg.norm(cen[j] - m) <= 1e-3 * max(np.linalg.norm(m), 1.0), f"cluster {j}"
