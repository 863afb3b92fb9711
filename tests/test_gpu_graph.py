"""The fit entry points under HIP graph capture.

kmeans_fit and kmeans_emeans enqueue kernels and device-to-device copies
only (no allocation, no host synchronization, no memset nodes: buffers are
cleared by fill kernels), so a caller can capture a whole fit into a graph
and replay it.  Each test captures a fit on torch's capture stream, then
replays the graph several times with other eager work and synchronizations
between the replays, and compares every replay with an eager run of the same
fit: bit for bit for kmeans_fit, up to the order of float additions for
e-means.
"""
import numpy as np
import pytest
import torch

import workloads
from tests import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def km():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_lloyd_means_03_amd as km
    km.load()
    return km


def _same(a, b, what, exact=False):
    """Two runs of the same fit.  kmeans_fit is a deterministic function of
    its inputs (stable sort, partial sums folded in a fixed order): exact
    equality.  e-means sorts each batch in the order labels arrive and folds
    partial sums with float atomics, so its centroids can differ in their
    last bits, and a point at a near tie can then change its label in a later
    step; counts and centroids are compared when the label sets agree."""
    if exact:
        for x, y, name in zip(a, b, ("centroids", "labels", "counts", "objective")):
            assert torch.equal(x, y), f"{what}: {name} differ"
        return
    (ca, la, na, ja), (cb, lb, nb, jb) = a, b
    assert (la != lb).float().mean().item() <= 1e-3, f"{what}: labels differ"
    np.testing.assert_allclose(ja.cpu().numpy(), jb.cpu().numpy(), rtol=1e-5, err_msg=what)
    if torch.equal(la, lb):
        assert torch.equal(na, nb), f"{what}: counts differ"
        parity.check_centroids(ca.cpu().numpy().reshape(1, -1, ca.shape[-1]),
                               cb.cpu().numpy().reshape(1, -1, cb.shape[-1]), what, rel=1e-5)


def _replays(graph, outs, eager, what, exact=False):
    for r in range(3):
        for t in outs:
            t.fill_(0)
        # other work on the default stream between replays
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        _same(tuple(t.clone() for t in outs), eager, f"{what}, replay {r}", exact)


def test_fit_in_a_graph(km):
    wl = workloads.small("gmm-n1m-k8192-d128-f16", N=20000, K=256, n_iter=3, seed=21)
    p = workloads.generate(wl)
    x, init = p.x.cuda(), p.init.cuda()
    B, N, d, K = wl.B, wl.N, wl.d, wl.K
    ws = km.workspace(B, N, d, K, x.dtype, x.device)
    eager = tuple(t.clone() for t in km.kmeans_fit(x, init, 3, ws=ws))
    torch.cuda.synchronize()

    cen = torch.empty_like(init)
    lab = torch.empty((B, N), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, K), dtype=torch.int32, device="cuda")
    obj = torch.empty((B, 3), dtype=torch.float64, device="cuda")
    # warm up on a side stream (torch's advice before capture), then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        km.kmeans_fit(x, init, 3, centroids=cen, labels=lab, counts=cnt, objective=obj, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        km.kmeans_fit(x, init, 3, centroids=cen, labels=lab, counts=cnt, objective=obj, ws=ws)
    _replays(g, (cen, lab, cnt, obj), eager, "kmeans_fit", exact=True)


def test_emeans_in_a_graph(km):
    N, d, K, batch, epochs = 30000, 32, 200, 4096, 2
    wl = workloads.small("gmm-n1m-k8192-d128-f16", N=N, d=d, K=K, n_iter=1, seed=22, ncomp=K // 2)
    p = workloads.generate(wl)
    x, init = p.x[0].cuda(), p.init[0].cuda()
    T = km.emeans_steps(N, batch, epochs)
    u = torch.from_numpy(workloads.emeans_uniforms(22, T, K)).cuda()
    L = km.load()
    ws = torch.empty(int(L.kmeans_emeans_workspace_bytes(N, d, K, 1, batch)), dtype=torch.uint8, device="cuda")
    args = (x, init, batch, epochs, 0.5, 0.1, 0.2, 1e-2)
    c0, l0, n0, j0 = km.kmeans_emeans(*args, uniforms=u, labels=True, ws=ws)
    eager = (c0.clone(), l0.clone(), n0.clone(), j0.clone())
    torch.cuda.synchronize()

    cen = torch.empty_like(init)
    lab = torch.empty((N,), dtype=torch.int32, device="cuda")
    cnt = torch.empty((K,), dtype=torch.int32, device="cuda")
    obj = torch.empty((T,), dtype=torch.float64, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        km.kmeans_emeans(*args, uniforms=u, centroids=cen, labels=lab, counts=cnt, objective=obj, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        km.kmeans_emeans(*args, uniforms=u, centroids=cen, labels=lab, counts=cnt, objective=obj, ws=ws)
    _replays(g, (cen, lab, cnt, obj), eager, "kmeans_emeans")


def test_emeans_sliced_and_short_paths_in_a_graph(km):
    """Batches of 2048 points against 4096 centroids: the assignment cuts the
    centroid tiles into slices and merges them, and the reduction takes the
    one-segment-per-row-group path chosen on the device by the sort's flag;
    both run inside the captured graph."""
    N, d, K, batch, epochs = 8192, 32, 4096, 2048, 2
    wl = workloads.small("gmm-n1m-k8192-d128-f16", N=N, d=d, K=K, n_iter=1, seed=23, ncomp=K // 4)
    p = workloads.generate(wl)
    x, init = p.x[0].cuda(), p.init[0].cuda()
    T = km.emeans_steps(N, batch, epochs)
    u = torch.from_numpy(workloads.emeans_uniforms(23, T, K)).cuda()
    L = km.load()
    ws = torch.empty(int(L.kmeans_emeans_workspace_bytes(N, d, K, 1, batch)), dtype=torch.uint8, device="cuda")
    args = (x, init, batch, epochs, 0.5, 0.1, 0.2, 1e-2)
    c0, l0, n0, j0 = km.kmeans_emeans(*args, uniforms=u, labels=True, ws=ws)
    eager = (c0.clone(), l0.clone(), n0.clone(), j0.clone())
    torch.cuda.synchronize()

    cen = torch.empty_like(init)
    lab = torch.empty((N,), dtype=torch.int32, device="cuda")
    cnt = torch.empty((K,), dtype=torch.int32, device="cuda")
    obj = torch.empty((T,), dtype=torch.float64, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        km.kmeans_emeans(*args, uniforms=u, centroids=cen, labels=lab, counts=cnt, objective=obj, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        km.kmeans_emeans(*args, uniforms=u, centroids=cen, labels=lab, counts=cnt, objective=obj, ws=ws)
    _replays(g, (cen, lab, cnt, obj), eager, "kmeans_emeans sliced + short")
