"""kmeans_fit_static (the fit that allocates nothing: its scratch is a static
per-device array) against kmeans_fit with a caller workspace, on two calls
in a row, the second on a smaller problem than the first, so the second
call finds the array holding the first call's data.

Both fits run the same kernels on the same inputs.  The bar is the one of
the oracle comparisons: labels equal except points the oracle flags as near
ties at the final centroids, counts consistent with the labels, centroids
within 1e-3 of the row scale, objectives within 1e-3 relative.  Each fit is
also compared with the oracle's fit of the same problem.
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


def _outputs(B, N, K, d, dev):
    return (torch.empty((B, K, d), dtype=torch.float32, device=dev),
            torch.empty((B, N), dtype=torch.int32, device=dev),
            torch.empty((B, K), dtype=torch.int32, device=dev))


def _case(km, wl):
    print(f"no-alloc: {wl.name} B={wl.B} N={wl.N} d={wl.d} K={wl.K} {wl.dtype} iters={wl.n_iter}", flush=True)
    p = workloads.generate(wl)
    x, w, init = parity.to_device(p)
    B, N, d, K, T = wl.B, wl.N, wl.d, wl.K, wl.n_iter
    C0, L0, n0 = _outputs(B, N, K, d, x.device)
    J0 = torch.empty((B, T), dtype=torch.float64, device=x.device)
    km.kmeans_fit(x, init, T, weights=w, centroids=C0, labels=L0, counts=n0, objective=J0)
    C1, L1, n1 = _outputs(B, N, K, d, x.device)
    J1 = torch.empty((B, T), dtype=torch.float64, device=x.device)
    km.kmeans_fit_static(x, init, T, weights=w, centroids=C1, labels=L1, counts=n1, objective=J1)
    torch.cuda.synchronize()
    C0, L0, n0, J0 = C0.cpu().numpy(), L0.cpu().numpy(), n0.cpu().numpy(), J0.cpu().numpy()
    C1, L1, n1, J1 = C1.cpu().numpy(), L1.cpu().numpy(), n1.cpu().numpy(), J1.cpu().numpy()

    # the two GPU fits against each other
    parity.check_centroids(C1, C0, f"{wl.name} static vs workspace centroids")
    parity.check_objective(J1, J0, f"{wl.name} static vs workspace objective")
    for b in range(B):
        np.testing.assert_array_equal(n1[b], np.bincount(L1[b], minlength=K))
    ref = oracle.fit(workloads.raw_bits(p.x), wl.dtype, None if p.w is None else p.w.numpy(), p.init.numpy(), T)
    parity.check_labels(L1, L0, ref["d1"], ref["d2"], f"{wl.name} static vs workspace labels")
    # and each against the oracle's fit
    for what, (C, L, J) in (("workspace", (C0, L0, J0)), ("static", (C1, L1, J1))):
        parity.check_centroids(C, ref["centroids"], f"{wl.name} {what} vs oracle")
        parity.check_objective(J, ref["J"], f"{wl.name} {what} vs oracle")
        parity.check_labels(L, ref["labels"], ref["d1"], ref["d2"], f"{wl.name} {what} vs oracle")


def test_static_fit_two_calls_second_smaller(km):
    big = workloads.small("gmm-n8192-k256-d128-f32", n_iter=6)
    small = workloads.small("gmm-b32-n65536-k1024-d128-f16", B=2, N=3001, K=97, n_iter=5)
    assert small.B * small.N < big.B * big.N and small.K < big.K
    _case(km, big)
    _case(km, small)


def test_static_fit_rejects_shapes_beyond_the_array(km):
    L = km.load()
    limit = int(L.kmeans_fit_static_max_bytes())
    assert limit == 64 << 20
    B, N, d, K = 1, 1 << 24, 128, 4096
    assert km.workspace_bytes(B, N, d, K, torch.float16) > limit
    # rejected on the host before any allocation or launch; the tensors are
    # never touched (a zero-stride view stands in for the large point tensor)
    x = torch.zeros((1, 1, d), dtype=torch.float16, device="cuda").expand(B, N, d)
    with pytest.raises(ValueError):
        km.kmeans_fit_static(x, torch.zeros((B, K, d), device="cuda"), 1)
    st = L.kmeans_fit_static(x.data_ptr(), 1, None, B, N, d, K, x.data_ptr(), 1, x.data_ptr(), None, None, None,
                             None)
    assert st == 3 and b"static" in L.kmeans_last_error()
