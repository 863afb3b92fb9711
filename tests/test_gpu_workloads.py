"""GPU parity at the full sizes of the measured workloads.

Protocol (teacher forced): the GPU runs a few Lloyd iterations to reach a
realistic iterate C_t; then
  * assignment at C_t: GPU labels and min_dist against the oracle on a seeded
    subsample of points (the oracle's N x K cost is too large for all points),
    and the GPU objective against the oracle's objective of the GPU labels
    over all points;
  * update with the GPU labels: counts exactly (all clusters) and centroids
    against the oracle (all clusters, or a sample of clusters that includes
    the largest one for the 33M-point workload).
The scalar-row workloads are small enough for a free-running comparison of
all 30 iterations.
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


def _log(msg):
    print(msg, flush=True)


def _teacher_forced(km, name, iters, n_sample, cluster_sample=None, chunk=1 << 20):
    wl = workloads.WORKLOADS[name]
    _log(f"[{name}] generating inputs")
    p = workloads.generate(wl)
    x, w, init = parity.to_device(p)
    B, N, d, K = wl.B, wl.N, wl.d, wl.K
    ws = km.workspace(B, N, d, K, x.dtype, x.device)
    _log(f"[{name}] GPU fit for {iters} iterations")
    C, _, _, J = km.kmeans_fit(x, init, iters, weights=w, ws=ws)
    labels, md, obj = km.kmeans_assign(x, C, weights=w, min_dist=True, objective=True, ws=ws)
    c_new, counts = km.kmeans_update(x, labels, C, weights=w, ws=ws)
    torch.cuda.synchronize()
    Ch = C.cpu().numpy()
    gl = labels.cpu().numpy()
    gmd = md.cpu().numpy()
    bits = workloads.raw_bits(p.x)
    Chat = oracle.decode(oracle.round_to(Ch, wl.dtype), wl.dtype)

    # --- assignment on a subsample
    _log(f"[{name}] oracle assignment on {n_sample} points per batch")
    rng = np.random.default_rng(2024)
    idx = np.sort(rng.choice(N, size=min(n_sample, N), replace=False))
    Xs = oracle.decode(bits[:, idx], wl.dtype)
    lab_ref, d1, d2 = oracle.assign(Xs, Chat)
    flips = parity.check_labels(gl[:, idx], lab_ref, d1, d2, f"{name} assign")
    parity.check_min_dist(gmd[:, idx], Xs, Chat, lab_ref, d1, f"{name} min_dist")

    # --- objective of the GPU labels over all points (chunked decode)
    _log(f"[{name}] oracle objective of the GPU labels")
    Jref = np.zeros(B)
    wn = None if p.w is None else p.w.numpy()
    for s in range(0, N, chunk):
        e = min(N, s + chunk)
        Xc = oracle.decode(bits[:, s:e], wl.dtype)
        Jref += oracle.objective(Xc, None if wn is None else wn[:, s:e], gl[:, s:e], Chat)
    parity.check_objective(obj.cpu().numpy(), Jref, f"{name} objective")

    # --- update with the GPU labels
    gc = c_new.cpu().numpy()
    gn = counts.cpu().numpy()
    for b in range(B):
        np.testing.assert_array_equal(gn[b], np.bincount(gl[b], minlength=K))
    if cluster_sample is None:
        _log(f"[{name}] oracle update, all points")
        X = oracle.decode(bits, wl.dtype)
        ref_c, ref_n, _, _ = oracle.update(X, wn, gl, Ch)
        np.testing.assert_array_equal(gn, ref_n)
        parity.check_centroids(gc, ref_c, f"{name} update")
    else:
        assert B == 1
        sizes = gn[0]
        rng = np.random.default_rng(7)
        pick = np.unique(np.concatenate([[int(np.argmax(sizes))],
                                         rng.choice(K, size=cluster_sample, replace=False)]))
        _log(f"[{name}] oracle update on {len(pick)} clusters ({int(sizes[pick].sum())} points)")
        relabel = np.full(K, -1, np.int64)
        relabel[pick] = np.arange(len(pick))
        mem = np.nonzero(relabel[gl[0]] >= 0)[0]
        Xp = oracle.decode(bits[:, mem], wl.dtype)
        ref_c, ref_n, _, _ = oracle.update(Xp, None if wn is None else wn[:, mem],
                                           relabel[gl[0, mem]][None].astype(np.int32), Ch[:, pick])
        np.testing.assert_array_equal(gn[:, pick], ref_n)
        # the tolerance's RMS floor is the full batch's, so compare against all rows
        full_ref = gc.copy()
        full_ref[:, pick] = ref_c
        parity.check_centroids(gc, full_ref, f"{name} update (sampled clusters)")
    _log(f"[{name}] ok, near-tie flips in the sample: {flips}")


def test_batched_b32_n65536_k1024_fp16(km):
    _teacher_forced(km, "gmm-b32-n65536-k1024-d128-f16", iters=3, n_sample=768)


def test_headline_n1m_k8192_fp16(km):
    _teacher_forced(km, "gmm-n1m-k8192-d128-f16", iters=3, n_sample=4096)


@pytest.mark.timeout(900)
def test_zipf_n32m_k4096_bf16(km):
    _teacher_forced(km, "zipf-n32m-k4096-d128-bf16", iters=2, n_sample=2048, cluster_sample=48)


@pytest.mark.parametrize("name", ["rows1d-b4096-n4096-k16-f32", "rows1d-b4096-n4096-k8-f32"])
def test_rows1d_full_fit(km, name):
    wl = workloads.WORKLOADS[name]
    p = workloads.generate(wl)
    x, w, init = parity.to_device(p)
    cen, lab, cnt, J = km.kmeans_fit(x, init, wl.n_iter, weights=w)
    torch.cuda.synchronize()
    ref = oracle.fit(workloads.raw_bits(p.x), wl.dtype, p.w.numpy(), p.init.numpy(), wl.n_iter)
    parity.check_objective(J.cpu().numpy(), ref["J"], name)
    parity.check_labels(lab.cpu().numpy(), ref["labels"], ref["d1"], ref["d2"], name)
    parity.check_centroids(cen.cpu().numpy(), ref["centroids"], name)
