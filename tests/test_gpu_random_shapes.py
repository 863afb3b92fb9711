"""GPU parity on seeded random shapes, to reach the launch rules (group
shapes, padded widths 16 … 512 including 96, piece widths, the direct and the
chunked label sort, the d = 1 paths) with combinations no hand-picked case
lists.  Each case runs the assignment against the oracle (labels up to near
ties, min_dist, objective), the update of random labels against the oracle
(counts exact, centroids per the Lloyd tolerance, empty clusters unchanged),
the label sort (segment sets exact) and one fit iteration (its labels and
objective like the assignment's, its update against the oracle's update of
the same labels).  The shapes are drawn from a fixed
seed, so every run checks the same cases.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import parity

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _cases(n=32, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = ["f32", "f16", "bf16"][i % 3]
        B = int(rng.choice([1, 1, 2, 3]))
        N = int(rng.integers(1, 3000))
        dmax = 256 if dtype == "f32" else 512
        d = int(rng.choice([1, 2, int(rng.integers(3, 17)), int(rng.integers(17, 65)), int(rng.integers(65, 97)),
                            int(rng.integers(97, 129)), int(rng.integers(129, dmax + 1))]))
        K = int(rng.choice([1, int(rng.integers(2, 17)), int(rng.integers(2, 17)), int(rng.integers(17, 300)),
                            int(rng.integers(17, 300)), int(rng.integers(300, 2500)), int(rng.integers(300, 2500))]))
        weighted = bool(rng.integers(0, 2))
        out.append((i, dtype, B, N, d, K, weighted))
    return out


@pytest.fixture(scope="module")
def km():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_lloyd_means_03_amd as km
    km.load()
    return km


@pytest.mark.parametrize("i,dtype,B,N,d,K,weighted", _cases())
def test_random_shape(km, i, dtype, B, N, d, K, weighted):
    what = f"case {i}: {dtype} B{B} N{N} d{d} K{K} w{weighted}"
    g = torch.Generator().manual_seed(1000 + i)
    x = torch.randn(B, N, d, generator=g).to(DT[dtype])
    C = torch.randn(B, K, d, generator=g)
    w = (torch.rand(B, N, generator=g) * 0.9 + 0.1) if weighted else None
    xd, Cd = x.cuda(), C.cuda()
    wd = None if w is None else w.cuda()

    # assignment
    labels, md, obj = km.kmeans_assign(xd, Cd, weights=wd, min_dist=True, objective=True)
    torch.cuda.synchronize()
    X, Chat, lab_ref, d1, d2 = parity.oracle_assign(workloads.raw_bits(x), dtype, C.numpy())
    parity.check_labels(labels.cpu().numpy(), lab_ref, d1, d2, what)
    parity.check_min_dist(md.cpu().numpy(), X, Chat, lab_ref, d1, what)
    wn = np.ones(d1.shape) if w is None else w.numpy().astype(np.float64)
    parity.check_objective(obj.cpu().numpy(), (wn * d1).sum(-1), what)

    # update of random labels (some clusters left empty)
    rng = np.random.default_rng(i)
    lab = rng.integers(0, max(1, K - K // 4), size=(B, N)).astype(np.int32)
    c_new, counts = km.kmeans_update(xd, torch.from_numpy(lab).cuda(), Cd, weights=wd)
    torch.cuda.synchronize()
    ref_c, ref_n, _, _ = oracle.update(X, None if w is None else w.numpy(), lab, C.numpy())
    np.testing.assert_array_equal(counts.cpu().numpy(), ref_n, err_msg=what)
    parity.check_centroids(c_new.cpu().numpy(), ref_c, what)
    empty = ref_n == 0
    np.testing.assert_array_equal(c_new.cpu().numpy()[empty], C.numpy()[empty], err_msg=what)

    # the label sort on its own
    cnt, off, perm = km.kmeans_sort_labels(torch.from_numpy(lab).cuda(), K)
    torch.cuda.synchronize()
    parity.check_perm(lab, K, cnt.cpu().numpy(), off.cpu().numpy(), perm.cpu().numpy())

    # one fit iteration: its assignment is the one above, its update that of
    # its own labels (teacher forced)
    cen, flab, fcnt, J = km.kmeans_fit(xd, Cd, 1, weights=wd)
    torch.cuda.synchronize()
    fl = flab.cpu().numpy()
    parity.check_labels(fl, lab_ref, d1, d2, what + " fit")
    parity.check_objective(J.cpu().numpy()[:, 0], (wn * d1).sum(-1), what + " fit")
    ref_c, ref_n, _, _ = oracle.update(X, None if w is None else w.numpy(), fl, C.numpy())
    np.testing.assert_array_equal(fcnt.cpu().numpy(), ref_n, err_msg=what + " fit")
    parity.check_centroids(cen.cpu().numpy(), ref_c, what + " fit")
