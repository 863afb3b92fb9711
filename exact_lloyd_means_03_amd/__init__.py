"""Exact Lloyd k-means for AMD Instinct MI355X (gfx950).

The computation lives in libkmeans_mi355x.so (hand-written HIP kernels behind
the C ABI of include/kmeans.h); this package only marshals torch tensors into
that ABI.
"""
from .api import (  # noqa: F401
    emeans_steps, kmeans_assign, kmeans_emeans, kmeans_fit, kmeans_fit_static, kmeans_fit_stream,
    kmeans_optimal_1d, kmeans_sort_labels, kmeans_update, workspace, workspace_bytes,
)
from ._lib import KMeansError, load  # noqa: F401

__all__ = ["emeans_steps", "kmeans_assign", "kmeans_emeans", "kmeans_fit", "kmeans_fit_static", "kmeans_fit_stream",
           "kmeans_optimal_1d", "kmeans_sort_labels", "kmeans_update", "workspace", "workspace_bytes",
           "KMeansError", "load"]
