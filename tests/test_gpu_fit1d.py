"""GPU parity of whole fits of scalar rows (d == 1) against the oracle.

Rows of up to 8192 points with K <= 16 run every iteration in one launch;
the cases below cover that path's edges (one centroid, duplicate centroids,
centroids a few floats apart, unweighted and weighted rows, ragged row
lengths, 16-bit points, rows of more than 4096 points, a single iteration,
optional outputs) and the boundary to the per-iteration path (K = 17, N = 8193), which must agree.
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


def _rows(B, N, K, dtype, weighted, seed, init="linspace"):
    rng = np.random.default_rng(seed)
    x32 = (0.02 * rng.standard_t(4.0, size=(B, N))).astype(np.float32)
    x = torch.from_numpy(x32).to(DT[dtype]).reshape(B, N, 1)
    w = torch.from_numpy(rng.uniform(0.1, 1.0, (B, N)).astype(np.float32)) if weighted else None
    xv = x.float().numpy()[..., 0]
    if init == "linspace":
        C = np.stack([np.linspace(r.min(), r.max(), K) for r in xv]).astype(np.float32)
    elif init == "dups":  # every value twice, in shuffled index order
        base = np.stack([np.linspace(r.min(), r.max(), (K + 1) // 2) for r in xv])
        C = np.concatenate([base, base], 1)[:, :K]
        C = C[:, rng.permutation(K)].astype(np.float32)
    else:  # first K points
        C = xv[:, :K].astype(np.float32).copy()
    return x, w, torch.from_numpy(np.ascontiguousarray(C, dtype=np.float32)).reshape(B, K, 1)


def _compare(km, x, w, init, n_iter, what):
    dt = workloads.dtype_name(x)
    xd, wd, Cd = x.cuda(), None if w is None else w.cuda(), init.cuda()
    cen, lab, cnt, J = km.kmeans_fit(xd, Cd, n_iter, weights=wd)
    torch.cuda.synchronize()
    ref = oracle.fit(workloads.raw_bits(x), dt, None if w is None else w.numpy(), init.numpy(), n_iter)
    gl = lab.cpu().numpy()
    flips = parity.check_labels(gl, ref["labels"], ref["d1"], ref["d2"], what)
    parity.check_objective(J.cpu().numpy(), ref["J"], what)
    if flips == 0:
        np.testing.assert_array_equal(cnt.cpu().numpy(), ref["counts"])
    parity.check_centroids(cen.cpu().numpy(), ref["centroids"], what)
    return cen, lab, cnt, J


@pytest.mark.parametrize("B,N,K,dtype,weighted,init,n_iter", [
    (64, 4096, 16, "f32", True, "linspace", 30),
    (64, 4096, 8, "f32", False, "linspace", 30),
    (37, 1000, 5, "f32", True, "first", 12),     # ragged row length
    (16, 8192, 16, "f32", True, "linspace", 10),  # 32 points per thread
    (16, 5000, 16, "f16", True, "linspace", 10),
    (16, 3000, 12, "bf16", False, "linspace", 10),
    (8, 777, 1, "f32", True, "first", 5),        # one centroid: the weighted mean
    (8, 2048, 16, "f32", True, "dups", 8),       # duplicate centroid values
    (8, 300, 16, "f32", False, "first", 1),      # a single iteration
    (4, 20, 16, "f32", False, "first", 4),       # K close to N
])
def test_fit_rows_parity(km, B, N, K, dtype, weighted, init, n_iter):
    x, w, C = _rows(B, N, K, dtype, weighted, seed=B * 7 + N + K, init=init)
    _compare(km, x, w, C, n_iter, f"rows B{B} N{N} K{K} {dtype} w{weighted} {init} it{n_iter}")


def test_duplicates_keep_their_value_and_get_no_points(km):
    """In the first iteration a centroid whose value a smaller index also
    holds gets no points and keeps its value (later it may differ and win)."""
    x, w, C = _rows(4, 2048, 16, "f32", True, seed=3, init="dups")
    cen, lab, cnt, _ = _compare(km, x, w, C, 1, "dups")
    Cn = C.numpy()[..., 0]
    cnt = cnt.cpu().numpy()
    for b in range(4):
        for j in range(16):
            if any(Cn[b, k] == Cn[b, j] for k in range(j)):  # a smaller index holds this value
                assert cnt[b, j] == 0
                assert cen.cpu().numpy()[b, j, 0] == Cn[b, j]


def test_optional_outputs_and_no_iterations(km):
    x, w, C = _rows(5, 1500, 9, "f32", True, seed=11)
    xd, wd, Cd = x.cuda(), w.cuda(), C.cuda()
    full = km.kmeans_fit(xd, Cd, 7, weights=wd)
    import ctypes
    from exact_lloyd_means_03_amd import _lib
    L = _lib.load()
    ws = km.workspace(5, 1500, 1, 9, xd.dtype, xd.device)
    cen = torch.empty_like(Cd)
    st = L.kmeans_fit(ctypes.c_void_p(xd.data_ptr()), 0, ctypes.c_void_p(wd.data_ptr()), 5, 1500, 1, 9,
                      ctypes.c_void_p(Cd.data_ptr()), 7, ctypes.c_void_p(cen.data_ptr()), None, None, None,
                      ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0
    assert torch.equal(cen, full[0])
    c0, _, _, _ = km.kmeans_fit(xd, Cd, 0, weights=wd)
    torch.cuda.synchronize()
    assert torch.equal(c0, Cd)


@pytest.mark.parametrize("n_iter", [1, 4])
def test_close_thresholds_count_compares(km, n_iter):
    """Four centroids a few floats apart put three thresholds within a span
    far below the width of one table bucket, so two of them share a bucket:
    that iteration ranks points by compares, and with one iteration so do
    the labels and counts."""
    x, w, C = _rows(12, 4096, 16, "f32", True, seed=29)
    Cn = C.numpy()[..., 0].copy()
    for b in range(Cn.shape[0]):
        v = np.float32(np.median(x.numpy()[b, :, 0]))
        for j in range(4):  # indices 3, 7, 11, 15 hold v and the next floats above it
            Cn[b, 4 * j + 3] = v
            v = np.nextafter(v, np.float32(np.inf))
    C = torch.from_numpy(Cn).reshape(C.shape)
    _compare(km, x, w, C, n_iter, f"close thresholds it{n_iter}")


@pytest.mark.parametrize("N,K", [(4096, 17), (8193, 16)])
def test_beyond_the_on_chip_limits(km, N, K):
    """Shapes just past the single-launch limits take the per-iteration path."""
    x, w, C = _rows(6, N, K, "f32", True, seed=N + K)
    _compare(km, x, w, C, 6, f"per-iteration N{N} K{K}")
