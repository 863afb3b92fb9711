"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Teacher-forced step parity: the GPU assignment and the oracle assignment get
the same centroids; the GPU update and the oracle update get the same
labels.  Free-running fits are compared where the oracle finishes quickly.
Inputs are the seeded workloads (reduced sizes, several tiles and ragged
tails) plus edge cases.
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


def _rand_problem(B, N, d, K, dtype, seed, spread=1.0):
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn(B, N, d, generator=g) * spread).to(DT[dtype])
    C = torch.randn(B, K, d, generator=g) * spread
    return x, C


def _assign_case(km, x, C, w=None, what=""):
    xd, Cd = x.cuda(), C.cuda()
    wd = None if w is None else w.cuda()
    labels, md, obj = km.kmeans_assign(xd, Cd, weights=wd, min_dist=True, objective=True)
    torch.cuda.synchronize()
    dt = workloads.dtype_name(x)
    X, Chat, lab_ref, d1, d2 = parity.oracle_assign(workloads.raw_bits(x), dt, C.numpy())
    gl = labels.cpu().numpy()
    parity.check_labels(gl, lab_ref, d1, d2, what)
    parity.check_min_dist(md.cpu().numpy(), X, Chat, lab_ref, d1, what)
    wn = np.ones(d1.shape) if w is None else w.numpy().astype(np.float64)
    parity.check_objective(obj.cpu().numpy(), (wn * d1).sum(-1), what)
    return gl


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("B,N,d,K", [
    (1, 1, 8, 1), (1, 300, 128, 64), (2, 1000, 128, 65), (1, 513, 100, 300),
    (3, 257, 16, 7), (1, 700, 2, 5), (1, 400, 33, 130), (1, 300, 200, 40), (1, 260, 256, 70),
    (1, 2049, 64, 1000),
    # 16-bit rows of 65..96 elements are padded to 96 (rotation-swizzled tiles)
    (1, 700, 96, 300), (2, 515, 80, 257), (1, 400, 65, 33), (1, 1200, 96, 600),
])
def test_assign_parity(km, dtype, B, N, d, K):
    x, C = _rand_problem(B, N, d, K, dtype, seed=B * 1000 + N + d + K)
    _assign_case(km, x, C, what=f"{dtype} B{B} N{N} d{d} K{K}")


@pytest.mark.parametrize("dtype,B,N,d,K", [
    ("f16", 1, 300001, 128, 700), ("bf16", 1, 262147, 96, 513), ("f32", 1, 300001, 128, 300),
    ("f16", 3, 90001, 256, 257), ("bf16", 2, 150001, 64, 1030),
])
def test_assign_parity_persistent_walk(km, dtype, B, N, d, K):
    """More point groups than the chip holds blocks at once: every block walks
    several groups (next group's first tile and points loaded during the
    current group's last tile and output write), checked on every point."""
    x, C = _rand_problem(B, N, d, K, dtype, seed=N + d + K)
    _assign_case(km, x, C, what=f"persistent {dtype} B{B} N{N} d{d} K{K}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("K", [1, 2, 8, 16, 100, 1024, 1500, 16384])
def test_assign_1d_parity(km, dtype, K):
    x, C = _rand_problem(3, 5000, 1, K, dtype, seed=K, spread=0.05)
    w = torch.rand(3, 5000) * 0.9 + 0.1
    _assign_case(km, x, C, w=w, what=f"1d {dtype} K{K}")


def test_assign_1d_rejects_huge_k(km):
    x = torch.zeros(1, 10, 1, device="cuda")
    with pytest.raises(km.KMeansError, match="K <= 16384"):
        km.kmeans_assign(x, torch.zeros(1, 16385, 1, device="cuda"))


def test_assign_1d_exact_ties(km):
    # x exactly halfway between two centroids; duplicated centroid values
    C = torch.tensor([[[0.0], [1.0], [1.0], [-1.0], [0.5]]])
    x = torch.tensor([[[0.25], [0.75], [-0.5], [1.0], [2.0], [-3.0], [0.5]]])
    labels, md, _ = km.kmeans_assign(x.cuda(), C.cuda(), min_dist=True)
    np.testing.assert_array_equal(labels.cpu().numpy()[0], [0, 1, 0, 1, 1, 3, 4])
    # -0 and +0 are the same value: the smaller index wins among all equidistant centroids
    C = torch.tensor([[[2.0], [-0.0], [0.0], [-2.0]]])
    x = torch.tensor([[[1.0], [-1.0], [0.0], [-0.0]]])
    labels, _, _ = km.kmeans_assign(x.cuda(), C.cuda())
    np.testing.assert_array_equal(labels.cpu().numpy()[0], [0, 1, 1, 1])


def test_duplicate_centroids_smallest_index(km):
    for dtype in ("f32", "f16", "bf16"):
        x, C = _rand_problem(1, 600, 128, 40, dtype, seed=7)
        C[0, 33] = C[0, 5]
        C[0, 39] = C[0, 5]
        gl = _assign_case(km, x, C, what=f"dup {dtype}")
        assert not np.any(gl == 33) and not np.any(gl == 39)


def test_points_equal_centroids(km):
    # every point is exactly a centroid (d = 0 up to rounding): labels are the identity
    for dtype in ("f32", "f16", "bf16"):
        x, _ = _rand_problem(1, 200, 64, 1, dtype, seed=3)
        C = x.float().clone()
        labels, md, _ = km.kmeans_assign(x.cuda(), C.cuda(), min_dist=True)
        np.testing.assert_array_equal(labels.cpu().numpy()[0], np.arange(200))
        assert torch.all(md >= 0)


def test_empty_inputs(km):
    x = torch.zeros(2, 0, 16, device="cuda", dtype=torch.float16)
    C = torch.randn(2, 5, 16, device="cuda")
    labels, _, obj = km.kmeans_assign(x, C, objective=True)
    assert labels.shape == (2, 0)
    assert torch.all(obj == 0)
    c_new, counts = km.kmeans_update(x, labels, C)
    assert torch.equal(c_new, C) and torch.all(counts == 0)
    cen, lab, cnt, J = km.kmeans_fit(x, C, 3)
    assert torch.equal(cen, C) and torch.all(J == 0)
    xb = torch.zeros(0, 10, 16, device="cuda", dtype=torch.float16)
    km.kmeans_fit(xb, torch.zeros(0, 4, 16, device="cuda"), 2)
    torch.cuda.synchronize()


def test_misaligned_points(km):
    # a view that starts one element into its storage: the kernels fall back to element loads
    for dtype in ("f16", "bf16", "f32"):
        base, C = _rand_problem(1, 300 * 64 + 1, 1, 20, dtype, seed=11)
        x = base.reshape(-1)[1:].reshape(1, 300, 64)
        xd = base.cuda().reshape(-1)[1:].reshape(1, 300, 64)
        assert xd.data_ptr() % 16 != 0
        C = torch.randn(1, 20, 64)
        labels, md, _ = km.kmeans_assign(xd, C.cuda(), min_dist=True)
        X, Chat, lab_ref, d1, d2 = parity.oracle_assign(workloads.raw_bits(x.contiguous()), dtype, C.numpy())
        parity.check_labels(labels.cpu().numpy(), lab_ref, d1, d2, "misaligned " + dtype)
        w = torch.ones(1, 300, device="cuda")
        c_new, counts = km.kmeans_update(xd, labels, C.cuda(), weights=w)
        ref_c, ref_n, _, _ = oracle.update(X, None, labels.cpu().numpy(), C.numpy())
        np.testing.assert_array_equal(counts.cpu().numpy(), ref_n)
        parity.check_centroids(c_new.cpu().numpy(), ref_c, "misaligned update " + dtype)


def test_sort_labels(km):
    rng = np.random.default_rng(0)
    for (B, N, K) in [(1, 1, 1), (2, 5000, 7), (1, 70000, 3000), (3, 40000, 16), (1, 100, 5000),
                      # one to eight cursor tables per scatter block, many chunks, ragged tails
                      (1, 300001, 32768), (2, 200003, 16384), (1, 1 << 20, 8192), (1, 2000003, 4096),
                      (5, 77777, 1000), (1, 65536, 16384), (1, 4097, 2)]:
        lab = rng.integers(0, K, size=(B, N)).astype(np.int32)
        lab[:, ::97] = -1            # unlabeled points
        lab[:, 5::101] = K + 3       # out of range
        counts, offsets, perm = km.kmeans_sort_labels(torch.from_numpy(lab).cuda(), K)
        parity.check_perm(lab, K, counts.cpu().numpy(), offsets.cpu().numpy(), perm.cpu().numpy())


def test_sort_labels_one_label_and_determinism(km):
    # every point in one cluster (one segment across all chunks), then a
    # repeat of a random sort: the same permutation bit for bit
    for K in (1, 5, 8192):
        lab = np.full((1, 500000), K - 1, np.int32)
        counts, offsets, perm = km.kmeans_sort_labels(torch.from_numpy(lab).cuda(), K)
        parity.check_perm(lab, K, counts.cpu().numpy(), offsets.cpu().numpy(), perm.cpu().numpy())
    lab = torch.from_numpy(np.random.default_rng(5).integers(0, 3000, size=(2, 400000)).astype(np.int32)).cuda()
    a = km.kmeans_sort_labels(lab, 3000)
    b = km.kmeans_sort_labels(lab, 3000)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_sort_labels_skewed(km):
    # Zipf-like sizes: most points in a few segments
    rng = np.random.default_rng(1)
    K = 4096
    p = np.arange(1, K + 1, dtype=np.float64) ** -1.2
    p /= p.sum()
    lab = rng.choice(K, size=(1, 300000), p=p).astype(np.int32)
    counts, offsets, perm = km.kmeans_sort_labels(torch.from_numpy(lab).cuda(), K)
    parity.check_perm(lab, K, counts.cpu().numpy(), offsets.cpu().numpy(), perm.cpu().numpy())


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("B,N,d,K,weighted", [
    (1, 5000, 128, 64, False), (2, 3000, 128, 300, True), (1, 20000, 16, 5, False),
    (1, 1000, 33, 50, True), (1, 4000, 2, 3, False), (1, 2000, 256, 17, False),
    (1, 100, 64, 500, False), (2, 9000, 1, 12, True), (1, 20000, 1, 300, False),
])
def test_update_parity(km, dtype, B, N, d, K, weighted):
    x, C = _rand_problem(B, N, d, K, dtype, seed=N + K + d)
    rng = np.random.default_rng(N + K)
    lab = rng.integers(0, max(1, K - K // 5), size=(B, N)).astype(np.int32)  # top clusters empty
    w = torch.from_numpy(rng.uniform(0.1, 1.0, (B, N)).astype(np.float32)) if weighted else None
    c_new, counts = km.kmeans_update(x.cuda(), torch.from_numpy(lab).cuda(), C.cuda(),
                                     weights=None if w is None else w.cuda())
    X = oracle.decode(workloads.raw_bits(x), dtype)
    ref_c, ref_n, _, _ = oracle.update(X, None if w is None else w.numpy(), lab, C.numpy())
    np.testing.assert_array_equal(counts.cpu().numpy(), ref_n)
    parity.check_centroids(c_new.cpu().numpy(), ref_c, f"update {dtype} B{B} N{N} d{d} K{K} w{weighted}")
    # empty clusters keep the old centroid bit for bit
    empty = ref_n == 0
    np.testing.assert_array_equal(c_new.cpu().numpy()[empty], C.numpy()[empty])


@pytest.mark.parametrize("dtype,d,weighted", [("bf16", 96, False), ("f16", 128, True), ("f32", 33, True),
                                              ("f16", 512, False), ("bf16", 7, False)])
@pytest.mark.parametrize("big", [0, 64, 65, 300])
def test_update_short_segments(km, dtype, d, weighted, big):
    """Few points per cluster (N = 4K on average): problems whose clusters all
    hold at most 64 points are reduced one segment per row group; a cluster
    of 65 or more points sends the problem to the piece kernels.  Two
    problems in one call, the second always short, so the per-problem choice
    is exercised both ways; one cluster of each problem is empty."""
    B, K = 2, 1000
    N = 4 * K
    x, C = _rand_problem(B, N, d, K, dtype, seed=d + big)
    rng = np.random.default_rng(d + big + 1)
    lab = rng.integers(1, K, size=(B, N)).astype(np.int32)  # cluster 0 empty ...
    if big:
        lab[0, :big] = 5  # ... except in the first problem, where cluster 5 gets at least `big` points
        lab[0, big:][lab[0, big:] == 5] = 6
    w = torch.from_numpy(rng.uniform(0.1, 1.0, (B, N)).astype(np.float32)) if weighted else None
    c_new, counts = km.kmeans_update(x.cuda(), torch.from_numpy(lab).cuda(), C.cuda(),
                                     weights=None if w is None else w.cuda())
    X = oracle.decode(workloads.raw_bits(x), dtype)
    ref_c, ref_n, _, _ = oracle.update(X, None if w is None else w.numpy(), lab, C.numpy())
    np.testing.assert_array_equal(counts.cpu().numpy(), ref_n)
    if big:
        assert ref_n[0, 5] == big
    parity.check_centroids(c_new.cpu().numpy(), ref_c, f"short segments {dtype} d{d} w{weighted} big{big}")
    empty = ref_n == 0
    assert empty[:, 0].all()
    np.testing.assert_array_equal(c_new.cpu().numpy()[empty], C.numpy()[empty])


@pytest.mark.parametrize("dtype,d,weighted", [("f16", 8, True), ("bf16", 6, False), ("f32", 12, True)])
def test_update_long_pieces(km, dtype, d, weighted):
    """Pieces longer than one staged chunk of 512 sorted rows: at 9M points the
    reduction takes pieces of 1024 rows, so every piece stages its indices
    twice and its batches run across the chunk boundary (16-byte rows at d = 8
    fp16 and d = 12 fp32, element-wise rows at d = 6 bf16).  Cluster sizes
    follow a power law, so segments range from empty to millions of rows."""
    B, N, K = 1, 9_000_000, 3000
    x, C = _rand_problem(B, N, d, K, dtype, seed=d + 21)
    rng = np.random.default_rng(d + 22)
    pk = np.arange(1, K + 1, dtype=np.float64) ** -1.1
    pk /= pk.sum()
    lab = rng.permutation(K)[rng.choice(K, size=(B, N), p=pk)].astype(np.int32)
    w = torch.from_numpy(rng.uniform(0.1, 1.0, (B, N)).astype(np.float32)) if weighted else None
    c_new, counts = km.kmeans_update(x.cuda(), torch.from_numpy(lab).cuda(), C.cuda(),
                                     weights=None if w is None else w.cuda())
    X = oracle.decode(workloads.raw_bits(x), dtype)
    ref_c, ref_n, _, _ = oracle.update(X, None if w is None else w.numpy(), lab, C.numpy())
    np.testing.assert_array_equal(counts.cpu().numpy(), ref_n)
    parity.check_centroids(c_new.cpu().numpy(), ref_c, f"long pieces {dtype} d{d} w{weighted}")
    empty = ref_n == 0
    np.testing.assert_array_equal(c_new.cpu().numpy()[empty], C.numpy()[empty])


@pytest.mark.parametrize("dtype,d,weighted", [("f16", 64, False), ("bf16", 128, True), ("f32", 16, True)])
def test_update_segments_aligned_to_pieces(km, dtype, d, weighted):
    """Segment starts on the reduction pieces' first rows, with empty clusters
    around them.  At N = 16384 the pieces hold 32 sorted rows; cluster sizes
    of 32 and 64 put segment starts exactly on piece starts (the piece then
    begins a segment and stores no continuation slot), empty clusters sit
    between them (a piece's first segment is the non-empty one after them),
    and sizes of 1, 31, 33 and a 1504-point cluster shift the alignment
    between runs of aligned segments and make segments span many pieces."""
    N, K = 16384, 700
    pattern = [32, 0, 32, 0, 0, 64, 1, 31, 32, 33, 0, 31, 64, 0, 32, 1504, 32, 0, 1, 63]
    sizes = []
    while sum(sizes) < N and len(sizes) < K:
        sizes.append(pattern[len(sizes) % len(pattern)])
    sizes[-1] -= sum(sizes) - N if sum(sizes) > N else 0
    if sum(sizes) < N:
        sizes[0] += N - sum(sizes)
    sizes += [0] * (K - len(sizes))
    assert sum(sizes) == N and len(sizes) == K
    rng = np.random.default_rng(d + 7)
    lab = np.repeat(np.arange(K, dtype=np.int32), sizes)
    lab = lab[rng.permutation(N)].reshape(1, N)
    x, C = _rand_problem(1, N, d, K, dtype, seed=d + 11)
    w = torch.from_numpy(rng.uniform(0.1, 1.0, (1, N)).astype(np.float32)) if weighted else None
    c_new, counts = km.kmeans_update(x.cuda(), torch.from_numpy(lab).cuda(), C.cuda(),
                                     weights=None if w is None else w.cuda())
    X = oracle.decode(workloads.raw_bits(x), dtype)
    ref_c, ref_n, _, _ = oracle.update(X, None if w is None else w.numpy(), lab, C.numpy())
    np.testing.assert_array_equal(counts.cpu().numpy(), ref_n)
    np.testing.assert_array_equal(ref_n[0], np.asarray(sizes))
    parity.check_centroids(c_new.cpu().numpy(), ref_c, f"aligned segments {dtype} d{d} w{weighted}")
    empty = ref_n == 0
    np.testing.assert_array_equal(c_new.cpu().numpy()[empty], C.numpy()[empty])


@pytest.mark.parametrize("dtype,d,weighted", [("bf16", 128, False), ("f16", 64, True), ("f32", 1, True)])
def test_update_parity_zipf_sizes(km, dtype, d, weighted):
    """Cluster sizes with a power-law tail: the largest segments span hundreds
    of reduction pieces, the smallest are empty or hold one point."""
    B, N, K = 1, 200000, 1000
    x, C = _rand_problem(B, N, d, K, dtype, seed=d + 11)
    rng = np.random.default_rng(d + 12)
    pk = np.arange(1, K + 1, dtype=np.float64) ** -1.2
    pk /= pk.sum()
    lab = rng.permutation(K)[rng.choice(K, size=(B, N), p=pk)].astype(np.int32)
    w = torch.from_numpy(rng.uniform(0.1, 1.0, (B, N)).astype(np.float32)) if weighted else None
    c_new, counts = km.kmeans_update(x.cuda(), torch.from_numpy(lab).cuda(), C.cuda(),
                                     weights=None if w is None else w.cuda())
    X = oracle.decode(workloads.raw_bits(x), dtype)
    ref_c, ref_n, _, _ = oracle.update(X, None if w is None else w.numpy(), lab, C.numpy())
    np.testing.assert_array_equal(counts.cpu().numpy(), ref_n)
    parity.check_centroids(c_new.cpu().numpy(), ref_c, f"zipf update {dtype} d{d} w{weighted}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("N,d,K", [(700, 300, 90), (530, 512, 300), (400, 257, 33)])
def test_wide_rows_parity(km, dtype, N, d, K):
    """Rows wider than 256 elements (16-bit points only): assignment, update
    and a short fit."""
    x, C = _rand_problem(1, N, d, K, dtype, seed=N + d + K)
    gl = _assign_case(km, x, C, what=f"wide assign {dtype} d{d}")
    c_new, counts = km.kmeans_update(x.cuda(), torch.from_numpy(gl).cuda(), C.cuda())
    X = oracle.decode(workloads.raw_bits(x), dtype)
    ref_c, ref_n, _, _ = oracle.update(X, None, gl, C.numpy())
    np.testing.assert_array_equal(counts.cpu().numpy(), ref_n)
    parity.check_centroids(c_new.cpu().numpy(), ref_c, f"wide update {dtype} d{d}")
    g = torch.Generator().manual_seed(d)
    init = x[:, torch.randperm(N, generator=g)[:K]].float().contiguous()
    cen, lab, cnt, J = km.kmeans_fit(x.cuda(), init.cuda(), 3)
    torch.cuda.synchronize()
    ref = oracle.fit(workloads.raw_bits(x), dtype, None, init.numpy(), 3)
    parity.check_objective(J.cpu().numpy(), ref["J"], f"wide fit {dtype} d{d}")
    parity.check_labels(lab.cpu().numpy(), ref["labels"], ref["d1"], ref["d2"], f"wide fit {dtype} d{d}")
    parity.check_centroids(cen.cpu().numpy(), ref["centroids"], f"wide fit {dtype} d{d}")


def test_float32_rows_above_256_are_rejected(km):
    x, C = _rand_problem(1, 100, 300, 10, "f32", seed=1)
    with pytest.raises(Exception):
        km.kmeans_assign(x.cuda(), C.cuda())


def test_update_in_place_and_invalid_labels(km):
    x, C = _rand_problem(1, 3000, 64, 20, "f16", seed=5)
    rng = np.random.default_rng(5)
    lab = rng.integers(0, 20, size=(1, 3000)).astype(np.int32)
    lab[0, ::7] = -2
    lab[0, 3::11] = 99
    Cd = C.cuda()
    c_new, counts = km.kmeans_update(x.cuda(), torch.from_numpy(lab).cuda(), Cd, c_new=Cd)
    valid = (lab >= 0) & (lab < 20)
    X = oracle.decode(workloads.raw_bits(x), "f16")
    keep = np.nonzero(valid[0])[0]
    ref_c, ref_n, _, _ = oracle.update(X[:, keep], None, lab[:, keep], C.numpy())
    np.testing.assert_array_equal(counts.cpu().numpy(), ref_n)
    parity.check_centroids(Cd.cpu().numpy(), ref_c, "in place")


def _fit_compare(km, p, n_iter=None, what=""):
    wl = p.wl
    n_iter = wl.n_iter if n_iter is None else n_iter
    x, w, init = parity.to_device(p)
    cen, lab, cnt, J = km.kmeans_fit(x, init, n_iter, weights=w)
    torch.cuda.synchronize()
    ref = oracle.fit(workloads.raw_bits(p.x), wl.dtype, None if p.w is None else p.w.numpy(),
                     p.init.numpy(), n_iter)
    nt = oracle.near_tie(ref["d1"], ref["d2"])
    gl = lab.cpu().numpy()
    flips = int(((gl != ref["labels"]) & nt).sum())
    parity.check_objective(J.cpu().numpy(), ref["J"], what)
    parity.check_labels(gl, ref["labels"], ref["d1"], ref["d2"], what)
    if flips == 0:
        np.testing.assert_array_equal(cnt.cpu().numpy(), ref["counts"])
    parity.check_centroids(cen.cpu().numpy(), ref["centroids"], what)
    return flips


def test_fit_parity_gmm_fp32_full(km):
    """The 8192-point, K=256, d=128 float32 mixture, all 10 iterations."""
    p = workloads.generate(workloads.WORKLOADS["gmm-n8192-k256-d128-f32"])
    _fit_compare(km, p, what="gmm-n8192 f32")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fit_parity_gmm_half(km, dtype):
    wl = workloads.small("gmm-b32-n65536-k1024-d128-f16", B=3, N=6000, K=96, dtype=dtype, n_iter=8)
    _fit_compare(km, workloads.generate(wl), what=f"gmm small {dtype}")


def test_fit_parity_rows1d(km):
    wl = workloads.small("rows1d-b4096-n4096-k16-f32", B=64)
    _fit_compare(km, workloads.generate(wl), what="rows1d K16")
    wl = workloads.small("rows1d-b4096-n4096-k8-f32", B=64)
    _fit_compare(km, workloads.generate(wl), what="rows1d K8")


def test_fit_resume_and_batch_independence(km):
    wl = workloads.small("gmm-b32-n65536-k1024-d128-f16", B=4, N=3000, K=40, n_iter=6)
    p = workloads.generate(wl)
    x, w, init = parity.to_device(p)
    c6, l6, n6, J6 = km.kmeans_fit(x, init, 6)
    c2, _, _, J2 = km.kmeans_fit(x, init, 2)
    c4, l4, n4, J4 = km.kmeans_fit(x, c2, 4)
    parity.check_centroids(c4.cpu().numpy(), c6.cpu().numpy(), "resume")
    parity.check_objective(torch.cat([J2, J4], 1).cpu().numpy(), J6.cpu().numpy(), "resume J")
    perm = torch.tensor([2, 0, 3, 1])
    cp, lp, np_, Jp = km.kmeans_fit(x[perm].contiguous(), init[perm].contiguous(), 6)
    parity.check_centroids(cp.cpu().numpy(), c6[perm.cuda()].cpu().numpy(), "batch permutation")
    parity.check_objective(Jp.cpu().numpy(), J6[perm.cuda()].cpu().numpy(), "batch permutation J")


def test_k_greater_than_n(km):
    x, C = _rand_problem(1, 50, 32, 200, "f16", seed=9)
    cen, lab, cnt, J = km.kmeans_fit(x.cuda(), C.cuda(), 3)
    ref = oracle.fit(workloads.raw_bits(x), "f16", None, C.numpy(), 3)
    parity.check_labels(lab.cpu().numpy(), ref["labels"], ref["d1"], ref["d2"], "K>N")
    parity.check_centroids(cen.cpu().numpy(), ref["centroids"], "K>N")
    assert int(cnt.sum()) == 50


# Few point groups against many centroid tiles: the launch cuts the tiles into
# slices (at least 8 tiles each) and merges each point's best over the slices.
@pytest.mark.parametrize("dtype,B,N,d,K,weighted", [
    ("f16", 1, 3000, 128, 4096, False),   # 6 groups, 16 tiles: 2 slices
    ("bf16", 1, 1500, 96, 16384, True),   # 64 tiles: 8 slices
    ("f16", 1, 1000, 512, 2048, False),   # 64-row tiles, one column block per wave: 4 slices
    ("f32", 1, 1000, 256, 1700, True),    # 28 tiles: slices of 10, 10 and 8
    ("f16", 3, 700, 64, 4096, True),      # several problems
    ("bf16", 1, 1, 128, 8192, False),     # one point
    ("f32", 2, 777, 61, 3000, False),     # padded rows, ragged groups
])
def test_assign_centroid_slices(km, dtype, B, N, d, K, weighted):
    what = f"slices {dtype} B{B} N{N} d{d} K{K} w{weighted}"
    x, C = _rand_problem(B, N, d, K, dtype, seed=N + d + K)
    w = torch.rand(B, N, generator=torch.Generator().manual_seed(K)) * 0.9 + 0.1 if weighted else None
    _assign_case(km, x, C, w, what)


def test_assign_centroid_slices_ties_across_slices(km):
    """The second half of the centroids repeats the first, so every point's
    best value is reached in both slices; the merged label is the smaller
    index, as the textbook scan in ascending centroid order gives."""
    B, N, d, K = 1, 2500, 128, 4096
    x, C = _rand_problem(B, N, d, K, "f16", seed=5)
    C[:, K // 2:] = C[:, :K // 2]
    x[0, :100] = C[0, 7:107].to(torch.float16)  # points exactly on centroids as well
    gl = _assign_case(km, x, C, None, "ties across slices")
    assert (gl < K // 2).all()


def test_fit_with_centroid_slices(km):
    """Two fit iterations on a sliced launch: the fused divide writes the
    tiles that the next sliced assignment reads."""
    x, C = _rand_problem(1, 3000, 128, 4096, "bf16", seed=11)
    xd, Cd = x.cuda(), C.cuda()
    c1, l1, n1, J1 = km.kmeans_fit(xd, Cd, 1)
    c2, l2, n2, J2 = km.kmeans_fit(xd, Cd, 2)
    torch.cuda.synchronize()
    X, Chat, lab_ref, d1, d2 = parity.oracle_assign(workloads.raw_bits(x), "bf16", C.numpy())
    parity.check_labels(l1.cpu().numpy(), lab_ref, d1, d2, "fit slices it 1")
    ref_c, ref_n, _, _ = oracle.update(X, None, l1.cpu().numpy(), C.numpy())
    np.testing.assert_array_equal(n1.cpu().numpy(), ref_n)
    parity.check_centroids(c1.cpu().numpy(), ref_c, "fit slices it 1")
    # the second iteration: the oracle's assignment at the GPU's first centroids
    X, Chat, lab_ref, d1, d2 = parity.oracle_assign(workloads.raw_bits(x), "bf16", c1.cpu().numpy())
    parity.check_labels(l2.cpu().numpy(), lab_ref, d1, d2, "fit slices it 2")
    parity.check_objective(J2.cpu().numpy()[:, 1], d1.sum(-1), "fit slices it 2")


@pytest.mark.parametrize("name,kw", [
    ("gmm-n1m-k8192-d128-f16", dict(N=200003, K=2048, n_iter=3)),
    ("zipf-n32m-k4096-d128-bf16", dict(N=1000003, K=512, n_iter=3)),
    ("gmm-b32-n65536-k1024-d128-f16", dict(B=8, N=30001, K=700, n_iter=3)),
    ("gmm-n8192-k256-d128-f32", dict(n_iter=4)),
])
def test_fit_is_deterministic(km, name, kw):
    """Two fits of the same inputs give bit-identical centroids, labels,
    counts and objectives: the label sort is stable, every segment and slot
    is summed in a fixed order, and the fold adds the slots in piece order
    (no float atomics on the Lloyd path)."""
    wl = workloads.small(name, **kw)
    p = workloads.generate(wl)
    x, w, init = parity.to_device(p)
    a = km.kmeans_fit(x, init, wl.n_iter, weights=w)
    b = km.kmeans_fit(x, init, wl.n_iter, weights=w)
    torch.cuda.synchronize()
    for u, v, what in zip(a, b, ("centroids", "labels", "counts", "objective")):
        assert torch.equal(u, v), f"{name}: {what} differ between two runs"
    # and a separate update call on the final labels, twice
    c1, n1 = km.kmeans_update(x, a[1], a[0], weights=w)
    c2, n2 = km.kmeans_update(x, a[1], a[0], weights=w)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(n1, n2)
