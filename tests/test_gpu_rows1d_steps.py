"""GPU parity of the single assignment and update steps on scalar rows (d == 1).

Rows with at most 16 centroids, N a multiple of 4 and aligned storage take
the one-wave-per-chunk kernels (thresholds in scalar registers for the
assignment, per-lane float64 bins for the update); other rows take the
binary search over sorted keys and the whole-row or sorted update.  The
cases cover both sides of every such boundary: K of 1, 3, 4, 5, 8, 9 and 16,
ragged chunks, rows longer than one chunk, N not a multiple of 4, storage
that starts one element in, labels outside [0, K), empty clusters, weighted
and unweighted rows, and all three point dtypes.
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


def _rows(B, N, K, dtype, seed):
    """Student-t rows (the quantization workload's shape) and K centroids
    spread over each row's range, with one duplicated value per row."""
    rng = np.random.default_rng(seed)
    x = torch.from_numpy((0.02 * rng.standard_t(4.0, size=(B, N, 1))).astype(np.float32)).to(DT[dtype])
    xv = x.float().numpy()[..., 0]
    C = np.stack([rng.uniform(r.min(), r.max(), K) for r in xv]).astype(np.float32)
    if K >= 3:
        C[:, K - 1] = C[:, 1]
    w = torch.from_numpy(rng.uniform(0.1, 1.0, (B, N)).astype(np.float32))
    return x, torch.from_numpy(C).reshape(B, K, 1), w


def _assign(km, xd, x, C, w, what):
    labels, md, obj = km.kmeans_assign(xd, C.cuda(), weights=None if w is None else w.cuda(),
                                       min_dist=True, objective=True)
    torch.cuda.synchronize()
    dt = workloads.dtype_name(x)
    X, Chat, lab_ref, d1, d2 = parity.oracle_assign(workloads.raw_bits(x), dt, C.numpy())
    parity.check_labels(labels.cpu().numpy(), lab_ref, d1, d2, what)
    parity.check_min_dist(md.cpu().numpy(), X, Chat, lab_ref, d1, what)
    wn = np.ones(d1.shape) if w is None else w.numpy().astype(np.float64)
    parity.check_objective(obj.cpu().numpy(), (wn * d1).sum(-1), what)
    # without the optional outputs the labels are the same
    lab2, _, _ = km.kmeans_assign(xd, C.cuda())
    torch.cuda.synchronize()
    assert torch.equal(lab2, labels)


def _update(km, xd, x, C, w, lab, what):
    c_new, counts = km.kmeans_update(xd, torch.from_numpy(lab).cuda(), C.cuda(),
                                     weights=None if w is None else w.cuda())
    torch.cuda.synchronize()
    X = oracle.decode(workloads.raw_bits(x), workloads.dtype_name(x))
    # a label outside [0, K) belongs to no cluster: the oracle sees each row's other points
    K = C.shape[1]
    ref_c, ref_n = np.empty(C.shape, np.float32), np.empty((C.shape[0], K), np.int64)
    for b in range(X.shape[0]):
        keep = (lab[b] >= 0) & (lab[b] < K)
        wb = None if w is None else w.numpy()[b:b + 1, keep]
        rc, rn, _, _ = oracle.update(X[b:b + 1, keep], wb, lab[b:b + 1, keep], C.numpy()[b:b + 1])
        ref_c[b], ref_n[b] = rc[0], rn[0]
    np.testing.assert_array_equal(counts.cpu().numpy(), ref_n)
    parity.check_centroids(c_new.cpu().numpy(), ref_c, what)
    empty = ref_n == 0
    np.testing.assert_array_equal(c_new.cpu().numpy()[empty], C.numpy()[empty])


CASES = [
    # B, N, K
    (4, 4096, 16),          # one full chunk per row
    (3, 2 * 4096 + 260, 8),  # two full chunks and a ragged one
    (5, 1000, 5),
    (2, 12, 9),             # one partial group
    (3, 777, 16),           # N not a multiple of 4: binary search and whole-row update
    (2, 4096, 4),
    (2, 4100, 3),
    (6, 256, 1),
    (1, 16384, 16),         # the longest row of the one-wave update
    (1, 16388, 16),         # one group longer: the sorted update
    (2, 9002, 12),          # N not a multiple of 4 and past the whole-row update: sorted
]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("B,N,K", CASES)
def test_assign_rows(km, dtype, B, N, K):
    x, C, w = _rows(B, N, K, dtype, seed=B * 100000 + N + K)
    what = f"assign 1d {dtype} B{B} N{N} K{K}"
    _assign(km, x.cuda(), x, C, w, what + " weighted")
    _assign(km, x.cuda(), x, C, None, what)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("B,N,K", CASES)
def test_update_rows(km, dtype, B, N, K):
    x, C, w = _rows(B, N, K, dtype, seed=B * 100000 + N + K + 1)
    rng = np.random.default_rng(N + K)
    lab = rng.integers(0, max(1, K - 1), size=(B, N)).astype(np.int32)  # the last cluster is empty
    lab[:, 3::97] = -1      # outside [0, K): no cluster gets these points
    lab[:, 5::101] = K + 2
    what = f"update 1d {dtype} B{B} N{N} K{K}"
    _update(km, x.cuda(), x, C, w, lab, what + " weighted")
    _update(km, x.cuda(), x, C, None, lab, what)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_rows_one_element_into_storage(km, dtype):
    """Aligned-row kernels are only taken for aligned storage: a view one
    element in gives the same results through the element-wise kernels."""
    B, N, K = 3, 4096, 16
    x, C, w = _rows(B, N + 1, K, dtype, seed=77)
    base = x.reshape(-1)
    xs = base[1:1 + B * N].reshape(B, N, 1).contiguous()
    xd = base.cuda()[1:1 + B * N].reshape(B, N, 1)
    assert xd.data_ptr() % 8 != 0
    w = w.reshape(-1)[:B * N].reshape(B, N).contiguous()
    _assign(km, xd, xs, C, w, f"misaligned assign {dtype}")
    lab = np.random.default_rng(5).integers(0, K, size=(B, N)).astype(np.int32)
    _update(km, xd, xs, C, w, lab, f"misaligned update {dtype}")
