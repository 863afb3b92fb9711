"""GPU-vs-oracle comparison helpers shared by the GPU tests.

Tolerances:
  * labels: equal, except points whose oracle top-2 gap (d2 - d1) is at most
    1e-4 * d1 (near ties), where either label is correct;
  * counts: equal (teacher forced: both sides get the same labels);
  * centroids: per row, ||c_gpu - c_ref|| <= 1e-3 * max(||c_ref||, rms_b), with
    rms_b the RMS row norm of the batch (elementwise relative error is
    meaningless for coordinates near zero);
  * objective: |J_gpu - J_ref| <= 1e-3 * J_ref;
  * per-point min_dist: float32 accumulation of d products, whose error is
    bounded by a few d * 2^-24 * (||x||^2 + ||c||^2), plus 1e-4 * d1 for a
    near-tie label choice.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads

U32 = 2.0 ** -24


def host_bits(x: torch.Tensor) -> np.ndarray:
    return workloads.raw_bits(x.detach().cpu())


def oracle_assign(x_bits: np.ndarray, dtype: str, C: np.ndarray):
    X = oracle.decode(x_bits, dtype)
    Chat = oracle.decode(oracle.round_to(C, dtype), dtype)
    labels, d1, d2 = oracle.assign(X, Chat)
    return X, Chat, labels, d1, d2


def check_labels(gpu_labels: np.ndarray, ref_labels: np.ndarray, d1, d2, what=""):
    nt = oracle.near_tie(d1, d2)
    bad = (gpu_labels != ref_labels) & ~nt
    n_bad = int(bad.sum())
    assert n_bad == 0, (f"{what}: {n_bad} non-near-tie label mismatches "
                        f"(first at {np.argwhere(bad)[:5].tolist()})")
    return int(((gpu_labels != ref_labels) & nt).sum())


def check_min_dist(gpu_md: np.ndarray, X: np.ndarray, Chat: np.ndarray, ref_labels, d1, what=""):
    d = X.shape[-1]
    xx = (X ** 2).sum(-1)
    cc = np.take_along_axis((Chat ** 2).sum(-1), ref_labels.astype(np.int64), axis=1)
    tol = 1e-4 * d1 + 4.0 * max(d, 16) * U32 * (xx + cc) + 1e-30
    err = np.abs(gpu_md.astype(np.float64) - d1)
    worst = float((err / tol).max()) if err.size else 0.0
    assert worst <= 1.0, f"{what}: min_dist error {worst:.3g} x tolerance"


def check_objective(gpu_J, ref_J, what=""):
    gpu_J = np.asarray(gpu_J, np.float64)
    ref_J = np.asarray(ref_J, np.float64)
    tol = 1e-3 * np.abs(ref_J) + 1e-12
    err = np.abs(gpu_J - ref_J)
    assert np.all(err <= tol), f"{what}: objective rel err {float((err / np.maximum(np.abs(ref_J), 1e-300)).max()):.3g}"


def check_centroids(gpu_C: np.ndarray, ref_C: np.ndarray, what="", rel=1e-3):
    gpu_C = np.asarray(gpu_C, np.float64)
    ref_C = np.asarray(ref_C, np.float64)
    rownorm = np.sqrt((ref_C ** 2).sum(-1))                 # [B, K]
    rms = np.sqrt((rownorm ** 2).mean(-1, keepdims=True))   # [B, 1]
    tol = rel * np.maximum(rownorm, rms) + 1e-30
    err = np.sqrt(((gpu_C - ref_C) ** 2).sum(-1))
    worst = float((err / tol).max()) if err.size else 0.0
    assert worst <= 1.0, f"{what}: centroid error {worst:.3g} x tolerance"


def check_perm(labels: np.ndarray, K: int, counts, offsets, perm):
    """Counting-sort outputs: counts and offsets exact, and perm the stable
    argsort of the labels in [0, K): ascending labels, and within a label the
    point indices in ascending order (a unique result, compared exactly with
    numpy's stable argsort).  Entries from offsets[K] on are not checked."""
    B, N = labels.shape
    for b in range(B):
        lab = labels[b]
        valid = (lab >= 0) & (lab < K)
        want_counts = np.bincount(lab[valid], minlength=K)
        np.testing.assert_array_equal(counts[b], want_counts)
        want_off = np.concatenate([[0], np.cumsum(want_counts)])
        np.testing.assert_array_equal(offsets[b], want_off)
        tot = int(want_off[-1])
        idx = np.nonzero(valid)[0]
        want = idx[np.argsort(lab[idx], kind="stable")]
        np.testing.assert_array_equal(perm[b, :tot], want)


def to_device(p: workloads.Problem, dev="cuda"):
    x = p.x.to(dev)
    w = None if p.w is None else p.w.to(dev)
    init = p.init.to(dev)
    return x, w, init
