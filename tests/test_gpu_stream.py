"""GPU parity of fits whose points stay in host memory (kmeans_fit_stream).

The points are copied to the GPU chunk by chunk in every iteration; the
result must be a Lloyd fit like kmeans_fit's.  One iteration is compared
with the oracle teacher-forced (the assignment from init up to near ties,
its objective, and the update of the GPU's own labels: counts exact,
centroids within tolerance).  Several iterations are compared with
kmeans_fit on the same points in device memory (the first assignment is the
same computation, so its labels and objective agree exactly; later
iterations agree up to fp32 summation order, so a near-tie flip may move a
few labels, and one moved label moves its clusters' centroids: centroids
and counts are compared when the label sets agree).  Cases: several
chunks with a ragged last one, one chunk, pinned and pageable host memory,
weights, the three dtypes, no iterations.
"""
import numpy as np
import pytest
import torch

import oracle
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


def _problem(N, d, K, dtype, weighted, seed):
    """A Gaussian-mixture problem (one batch) and, if asked, U(0.1, 1) weights."""
    wl = workloads.small("gmm-b32-n65536-k1024-d128-f16", B=1, N=N, d=d, K=K, dtype=dtype, n_iter=5, seed=seed)
    p = workloads.generate(wl)
    w = None
    if weighted:
        w = torch.from_numpy(np.random.default_rng(seed).uniform(0.1, 1.0, (1, N)).astype(np.float32))
    return p.x, w, p.init


@pytest.mark.parametrize("dtype,d,weighted,chunk,pinned", [
    ("f16", 128, False, 8192, True),
    ("bf16", 64, True, 4096, True),
    ("f32", 33, True, 8192, False),
    ("f16", 128, True, 1 << 20, True),   # one chunk
])
def test_stream_fit_parity(km, dtype, d, weighted, chunk, pinned):
    N, K, n_iter = 30000, 64, 5
    x, w, init0 = _problem(N, d, K, dtype, weighted, seed=N + d + K)
    what = f"stream {dtype} d{d} w{weighted} chunk{chunk} pinned{pinned}"
    xh = x[0].contiguous()
    wh = None if w is None else w[0].contiguous()
    if pinned:
        xh = xh.pin_memory()
        wh = None if wh is None else wh.pin_memory()
    init = init0[0].cuda()
    wn = None if w is None else w.numpy()

    # one iteration against the oracle, teacher-forced: the assignment from
    # init, then the update of the GPU's own labels
    cen1, lab1, cnt1, J1 = km.kmeans_fit_stream(xh, init, 1, weights=wh, chunk=chunk, labels=True)
    torch.cuda.synchronize()
    X, Chat, lab_ref, d1, d2 = parity.oracle_assign(workloads.raw_bits(x), dtype, init0.numpy())
    gl = lab1.cpu().numpy()[None]
    parity.check_labels(gl, lab_ref, d1, d2, what)
    parity.check_objective(J1.cpu().numpy(), ((1.0 if wn is None else wn.astype(np.float64)) * d1).sum(-1), what)
    ref_c, ref_n, _, _ = oracle.update(X, wn, gl, init0.numpy())
    np.testing.assert_array_equal(cnt1.cpu().numpy()[None], ref_n)
    parity.check_centroids(cen1.cpu().numpy()[None], ref_c, what)

    # several iterations against the fit of the same points in device memory:
    # the same Lloyd iterations up to fp32 summation order
    cen, lab, cnt, J = km.kmeans_fit_stream(xh, init, n_iter, weights=wh, chunk=chunk, labels=True)
    x_dev = x.cuda()
    w_dev = None if w is None else w.cuda()
    cf, lf, nf, Jf = km.kmeans_fit(x_dev, init0.cuda(), n_iter, weights=w_dev)
    _, lab_f1, _, J_f1 = km.kmeans_fit(x_dev, init0.cuda(), 1, weights=w_dev)
    torch.cuda.synchronize()
    assert torch.equal(lab_f1[0], lab1), "the first assignment is the same computation"
    assert abs(J_f1[0, 0].item() - J1[0].item()) <= 1e-9 * abs(J_f1[0, 0].item())
    np.testing.assert_allclose(J.cpu().numpy(), Jf[0].cpu().numpy(), rtol=1e-5)
    assert (lab != lf[0]).float().mean().item() <= 1e-3, what
    if torch.equal(lab, lf[0]):
        # the same trajectory: counts equal, centroids equal up to summation order
        assert torch.equal(cnt, nf[0])
        parity.check_centroids(cen.cpu().numpy()[None], cf.cpu().numpy(), what)


def test_stream_fit_centroid_slices(km):
    """Chunks of 4096 points (8 groups) and a last chunk of 100 points
    against 4096 centroids: both assignments cut the centroid tiles into
    slices, and the last chunk's slices use the scratch sized for it."""
    N, d, K, chunk = 2 * 4096 + 100, 128, 4096, 4096
    x, _, init0 = _problem(N, d, K, "f16", False, seed=3)
    xh = x[0].contiguous().pin_memory()
    init = init0[0].cuda()
    cen1, lab1, cnt1, J1 = km.kmeans_fit_stream(xh, init, 1, chunk=chunk, labels=True)
    torch.cuda.synchronize()
    X, Chat, lab_ref, d1, d2 = parity.oracle_assign(workloads.raw_bits(x), "f16", init0.numpy())
    gl = lab1.cpu().numpy()[None]
    parity.check_labels(gl, lab_ref, d1, d2, "stream slices")
    parity.check_objective(J1.cpu().numpy(), d1.sum(-1), "stream slices")
    ref_c, ref_n, _, _ = oracle.update(X, None, gl, init0.numpy())
    np.testing.assert_array_equal(cnt1.cpu().numpy()[None], ref_n)
    parity.check_centroids(cen1.cpu().numpy()[None], ref_c, "stream slices")
    _, lab_f1, _, J_f1 = km.kmeans_fit(x.cuda(), init0.cuda(), 1)
    torch.cuda.synchronize()
    assert torch.equal(lab_f1[0], lab1), "the first assignment is the same computation"


def test_stream_fit_no_iterations_and_no_labels(km):
    x, _, init0 = _problem(10000, 32, 16, "f16", False, seed=5)
    xh = x[0].contiguous().pin_memory()
    init = init0[0].cuda()
    cen, lab, cnt, J = km.kmeans_fit_stream(xh, init, 0, chunk=4096)
    torch.cuda.synchronize()
    assert torch.equal(cen, init) and lab is None and J.numel() == 0
    cen2, _, _, J2 = km.kmeans_fit_stream(xh, init, 3, chunk=4096)
    cen3, lab3, _, J3 = km.kmeans_fit_stream(xh, init, 3, chunk=4096, labels=True)
    torch.cuda.synchronize()
    # with or without a label output the same fit (the labels then stay in the workspace)
    np.testing.assert_allclose(J2.cpu().numpy(), J3.cpu().numpy(), rtol=1e-6)
    parity.check_centroids(cen2.cpu().numpy()[None], cen3.cpu().numpy()[None], "labels or not")


def test_stream_fit_rejects_scalar_points(km):
    x = torch.zeros(100, 1)
    with pytest.raises(km.KMeansError, match="d >= 2"):
        km.kmeans_fit_stream(x, torch.zeros(4, 1, device="cuda"), 2)
