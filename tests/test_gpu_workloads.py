"""GPU parity at the full sizes of the measured workloads, every iteration.

Protocol (teacher forced, iteration by iteration): the GPU runs the
workload's Lloyd iterations one kmeans_fit call at a time, from the
workload's init, keeping every iterate C_t, the labels L_t of assignment t
and the counts, objective and centroids C_{t+1} of update t.  Then, for
every t:
  * assignment at C_t: GPU labels against the oracle's assignment at the same
    C_t, equal except near ties (the oracle's top-2 gap at most 1e-4 of the
    nearest distance); on all points where the oracle affords it, else on a
    fresh seeded sample of 65536 points per iteration, plus all points at one
    iterate.  min_dist of a separate kmeans_assign call on the same points;
  * objective: J_t against the oracle's sum over all points of the distance
    to the GPU's label (and, where every label was checked, against the sum
    of the oracle's nearest distances);
  * update with L_t: counts exactly, and C_{t+1} against the oracle's update
    of all points with L_t from C_t (per-row tolerance 1e-3 of the row scale).
The batched workload is also fitted free running (the fused path of
kmeans_fit, all 20 iterations in one call) and compared with the oracle's
own fit on several whole batches.  The scalar-row workloads are compared free
running over all 30 iterations.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import parity

pytestmark = pytest.mark.gpu

SAMPLE = 65536


@pytest.fixture(scope="module")
def km():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_lloyd_means_03_amd as km
    km.load()
    return km


def _log(msg):
    print(msg, flush=True)


class Trajectory:
    """A workload's GPU iterates, one kmeans_fit call per iteration."""

    def __init__(self, km, name, iters):
        wl = workloads.WORKLOADS[name]
        self.wl, self.name, self.iters = wl, name, iters
        _log(f"[{name}] generating inputs")
        p = workloads.generate(wl)
        self.bits = workloads.raw_bits(p.x)
        self.w = None if p.w is None else p.w.numpy()
        x, w, init = parity.to_device(p)
        B, N, d, K = wl.B, wl.N, wl.d, wl.K
        ws = km.workspace(B, N, d, K, x.dtype, x.device)
        self.C = [p.init.numpy()]              # C_0 .. C_iters (fp32, host)
        self.L, self.cnt, self.J = [], [], []  # per iteration: labels, counts, objective
        self.sample = []                       # per iteration: sampled indices, GPU min_dist there
        C = init
        for t in range(iters):
            _log(f"[{name}] GPU iteration {t}")
            Cn, L, n, J = km.kmeans_fit(x, C, 1, weights=w, ws=ws)
            L2, md, _ = km.kmeans_assign(x, C, weights=w, min_dist=True, ws=ws)
            torch.cuda.synchronize()
            Lh = L.cpu().numpy()
            # the fit's assignment and the assignment call run the same kernel
            # on the same centroids
            assert torch.equal(L, L2), f"{name}: fit and assign labels differ at t={t}"
            idx = self._sample_idx(t)
            self.sample.append((idx, md.cpu().numpy()[:, idx] if idx is not None else md.cpu().numpy()))
            self.L.append(Lh)
            self.cnt.append(n.cpu().numpy())
            self.J.append(J.cpu().numpy()[:, 0])
            self.C.append(Cn.cpu().numpy())
            C = Cn
        del x, w, ws
        torch.cuda.empty_cache()

    def _sample_idx(self, t):
        N = self.wl.N
        if N <= SAMPLE:
            return None
        return np.sort(np.random.default_rng(1000 + t).choice(N, size=SAMPLE, replace=False))

    def chat(self, t):
        return oracle.decode(oracle.round_to(self.C[t], self.wl.dtype), self.wl.dtype)


def _check_assign_sample(tr, t, batches=None):
    """Labels and min_dist of assignment t against the oracle, on the sample
    (all points when the problem is small), in the given batches (all)."""
    wl = tr.wl
    idx, md = tr.sample[t]
    bsel = slice(None) if batches is None else batches
    bits = tr.bits[bsel] if idx is None else tr.bits[bsel][:, idx]
    X = oracle.decode(bits, wl.dtype)
    Chat = tr.chat(t)[bsel]
    lab, d1, d2 = oracle.assign(X, Chat)
    gl = tr.L[t][bsel] if idx is None else tr.L[t][bsel][:, idx]
    flips = parity.check_labels(gl, lab, d1, d2, f"{tr.name} assign t={t}")
    parity.check_min_dist(md[bsel], X, Chat, lab, d1, f"{tr.name} min_dist t={t}")
    return flips, d1


def _check_update(tr, t):
    """Update t with the GPU's labels L_t, on all points."""
    wl = tr.wl
    K = wl.K
    for b in range(wl.B):
        np.testing.assert_array_equal(tr.cnt[t][b], np.bincount(tr.L[t][b], minlength=K))
    ref_c, ref_n, _, _ = oracle.update_bits(tr.bits, wl.dtype, tr.w, tr.L[t], tr.C[t])
    np.testing.assert_array_equal(tr.cnt[t], ref_n)
    parity.check_centroids(tr.C[t + 1], ref_c, f"{tr.name} update t={t}")


def _check_objective_of_labels(tr, t):
    J = oracle.objective_bits(tr.bits, tr.wl.dtype, tr.w, tr.L[t], tr.chat(t))
    parity.check_objective(tr.J[t], J, f"{tr.name} objective t={t}")


def _check_all_labels(tr, t, chunk=1 << 18):
    """Every label of assignment t, and J_t against the sum of the oracle's
    nearest distances."""
    wl = tr.wl
    Chat = tr.chat(t)
    Jref = np.zeros(wl.B)
    flips = 0
    for s in range(0, wl.N, chunk):
        e = min(wl.N, s + chunk)
        X = oracle.decode(tr.bits[:, s:e], wl.dtype)
        lab, d1, d2 = oracle.assign(X, Chat)
        flips += parity.check_labels(tr.L[t][:, s:e], lab, d1, d2, f"{tr.name} all labels t={t} [{s}:{e})")
        Jref += (d1 if tr.w is None else tr.w[:, s:e] * d1).sum(-1)
    parity.check_objective(tr.J[t], Jref, f"{tr.name} objective (oracle labels) t={t}")
    return flips


# ------------------------------------------------------------------ c3: N=1M

@pytest.fixture(scope="module")
def headline(km):
    return Trajectory(km, "gmm-n1m-k8192-d128-f16", iters=10)


@pytest.mark.timeout(600)
def test_headline_assign_every_iteration(headline):
    for t in range(headline.iters):
        flips, _ = _check_assign_sample(headline, t)
        _log(f"[headline] t={t}: {SAMPLE} sampled labels ok, near-tie flips {flips}")


@pytest.mark.timeout(600)
def test_headline_update_and_objective_every_iteration(headline):
    for t in range(headline.iters):
        _check_update(headline, t)
        _check_objective_of_labels(headline, t)
    _log("[headline] update and objective ok at every iteration")


@pytest.mark.timeout(600)
def test_headline_all_labels_one_iterate(headline):
    # the last iterate: every point through the persistent multi-group walk
    t = headline.iters - 1
    flips = _check_all_labels(headline, t)
    _log(f"[headline] all {headline.wl.N} labels ok at t={t}, near-tie flips {flips}")


# ------------------------------------------------- c2: B=32 x N=65536

C2 = "gmm-b32-n65536-k1024-d128-f16"
C2_BATCHES = [0, 9, 22, 31]


@pytest.fixture(scope="module")
def batched(km):
    return Trajectory(km, C2, iters=workloads.WORKLOADS[C2].n_iter)


@pytest.mark.timeout(600)
def test_batched_all_points_of_four_batches_every_iteration(batched):
    for t in range(batched.iters):
        flips, _ = _check_assign_sample(batched, t, batches=C2_BATCHES)
        _check_update(batched, t)
        _check_objective_of_labels(batched, t)
        _log(f"[batched] t={t}: batches {C2_BATCHES} all labels ok (flips {flips}), update ok")


@pytest.mark.timeout(600)
def test_batched_all_batches_one_iterate(batched):
    t = batched.iters // 2
    flips = _check_all_labels(batched, t)
    _log(f"[batched] all 32 x 65536 labels ok at t={t}, near-tie flips {flips}")


@pytest.mark.timeout(600)
def test_batched_free_running_fit(km):
    """The fused kmeans_fit (divide + next prep in one kernel, no host sync)
    over all 20 iterations of all 32 batches, against the oracle's own fit of
    four whole batches (batches are independent problems)."""
    wl = workloads.WORKLOADS[C2]
    p = workloads.generate(wl)
    x, w, init = parity.to_device(p)
    cen, lab, cnt, J = km.kmeans_fit(x, init, wl.n_iter)
    torch.cuda.synchronize()
    sel = C2_BATCHES
    bits = workloads.raw_bits(p.x)[sel]
    _log(f"[batched] oracle fit of batches {sel}, {wl.n_iter} iterations")
    ref = oracle.fit(bits, wl.dtype, None, p.init.numpy()[sel], wl.n_iter)
    parity.check_objective(J.cpu().numpy()[sel], ref["J"], "batched free-running objective")
    parity.check_labels(lab.cpu().numpy()[sel], ref["labels"], ref["d1"], ref["d2"], "batched free-running labels")
    parity.check_centroids(cen.cpu().numpy()[sel], ref["centroids"], "batched free-running centroids")
    np.testing.assert_array_equal(cnt.cpu().numpy()[sel].sum(-1), wl.N)


# ---------------------------------------------------- c4: N=32M, Zipf sizes

@pytest.fixture(scope="module")
def zipf(km):
    return Trajectory(km, "zipf-n32m-k4096-d128-bf16", iters=workloads.WORKLOADS["zipf-n32m-k4096-d128-bf16"].n_iter)


@pytest.mark.timeout(900)
def test_zipf_assign_every_iteration(zipf):
    for t in range(zipf.iters):
        flips, _ = _check_assign_sample(zipf, t)
        _log(f"[zipf] t={t}: {SAMPLE} sampled labels ok, near-tie flips {flips}")


@pytest.mark.timeout(900)
def test_zipf_update_all_clusters_every_iteration(zipf):
    for t in range(zipf.iters):
        _check_update(zipf, t)
        _log(f"[zipf] t={t}: update of all {zipf.wl.K} clusters ok (largest {int(zipf.cnt[t].max())} points)")


@pytest.mark.timeout(900)
def test_zipf_objective_every_iteration(zipf):
    for t in range(zipf.iters):
        _check_objective_of_labels(zipf, t)
    _log("[zipf] objective ok at every iteration")


# ------------------------------------------------ c5: scalar rows, d = 1

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
    gl, gc = lab.cpu().numpy(), cnt.cpu().numpy()
    for b in range(wl.B):
        np.testing.assert_array_equal(gc[b], np.bincount(gl[b], minlength=wl.K))
