"""Python entry points with the C ABI's names (argument marshalling only).

Tensors are torch tensors on the GPU: torch provides the device memory and
the stream (the current stream of the tensors' device).  Every step of the
computation runs in the HIP kernels of libkmeans_mi355x.so.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib

_DT = {torch.float32: _lib.KM_F32, torch.float16: _lib.KM_F16, torch.bfloat16: _lib.KM_BF16}


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dev_tensor(t, name, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _points(x):
    _dev_tensor(x, "x")
    if x.dim() != 3:
        raise ValueError("x must be [B, N, d]")
    if x.dtype not in _DT:
        raise TypeError(f"x dtype {x.dtype} is not float32 / float16 / bfloat16")
    return x.shape


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def workspace_bytes(B: int, N: int, d: int, K: int, dtype: torch.dtype) -> int:
    n = _lib.load().kmeans_workspace_bytes(B, N, d, K, _DT[dtype])
    if n == 0 and B * N * d * K > 0:
        _lib.check(2, "kmeans_workspace_bytes")
    return int(n)


def workspace(B: int, N: int, d: int, K: int, dtype: torch.dtype, device) -> torch.Tensor:
    """A device workspace large enough for every entry point at these shapes."""
    n = workspace_bytes(B, N, d, K, dtype)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _ws(ws, B, N, d, K, dtype, device):
    if ws is None:
        ws = workspace(B, N, d, K, dtype, device)
    _dev_tensor(ws, "workspace", torch.uint8)
    return ws


def kmeans_assign(x, centroids, weights=None, labels=None, min_dist=None, objective=None, ws=None):
    """Nearest centroid of every point.  Returns (labels, min_dist, objective);
    min_dist / objective are None unless tensors are passed in (or True)."""
    B, N, d = _points(x)
    _dev_tensor(centroids, "centroids", torch.float32)
    if centroids.dim() != 3 or centroids.shape[0] != B or centroids.shape[2] != d:
        raise ValueError("centroids must be [B, K, d] float32")
    K = centroids.shape[1]
    dev = x.device
    if weights is not None:
        _dev_tensor(weights, "weights", torch.float32, (B, N))
    labels = torch.empty((B, N), dtype=torch.int32, device=dev) if labels is None else \
        _dev_tensor(labels, "labels", torch.int32, (B, N))
    if min_dist is True:
        min_dist = torch.empty((B, N), dtype=torch.float32, device=dev)
    elif min_dist is not None:
        _dev_tensor(min_dist, "min_dist", torch.float32, (B, N))
    if objective is True:
        objective = torch.empty((B,), dtype=torch.float64, device=dev)
    elif objective is not None:
        _dev_tensor(objective, "objective", torch.float64, (B,))
    ws = _ws(ws, B, N, d, K, x.dtype, dev)
    st = _lib.load().kmeans_assign(_ptr(x), _DT[x.dtype], B, N, d, _ptr(centroids), K, _ptr(weights),
                                   _ptr(labels), _ptr(min_dist), _ptr(objective), _ptr(ws), ws.numel(),
                                   _stream(dev))
    _lib.check(st, "kmeans_assign")
    return labels, min_dist, objective


def kmeans_sort_labels(labels, K: int, ws=None):
    """Counting argsort of labels [B, N] int32.  Returns (counts, offsets, perm)."""
    _dev_tensor(labels, "labels", torch.int32)
    if labels.dim() != 2:
        raise ValueError("labels must be [B, N]")
    B, N = labels.shape
    dev = labels.device
    counts = torch.empty((B, K), dtype=torch.int32, device=dev)
    offsets = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    perm = torch.empty((B, N), dtype=torch.int32, device=dev)
    ws = _ws(ws, B, N, 2, K, torch.float32, dev)
    st = _lib.load().kmeans_sort_labels(_ptr(labels), B, N, K, _ptr(counts), _ptr(offsets), _ptr(perm),
                                        _ptr(ws), ws.numel(), _stream(dev))
    _lib.check(st, "kmeans_sort_labels")
    return counts, offsets, perm


def kmeans_update(x, labels, c_old, weights=None, c_new=None, counts=None, ws=None):
    """Centroids as the (weighted) means of their points; empty clusters keep
    c_old.  Returns (c_new, counts)."""
    B, N, d = _points(x)
    _dev_tensor(labels, "labels", torch.int32, (B, N))
    _dev_tensor(c_old, "c_old", torch.float32)
    if c_old.dim() != 3 or c_old.shape[0] != B or c_old.shape[2] != d:
        raise ValueError("c_old must be [B, K, d] float32")
    K = c_old.shape[1]
    dev = x.device
    if weights is not None:
        _dev_tensor(weights, "weights", torch.float32, (B, N))
    c_new = torch.empty_like(c_old) if c_new is None else _dev_tensor(c_new, "c_new", torch.float32, c_old.shape)
    counts = torch.empty((B, K), dtype=torch.int32, device=dev) if counts is None else \
        _dev_tensor(counts, "counts", torch.int32, (B, K))
    ws = _ws(ws, B, N, d, K, x.dtype, dev)
    st = _lib.load().kmeans_update(_ptr(x), _DT[x.dtype], _ptr(weights), B, N, d, _ptr(labels), K,
                                   _ptr(c_old), _ptr(c_new), _ptr(counts), _ptr(ws), ws.numel(), _stream(dev))
    _lib.check(st, "kmeans_update")
    return c_new, counts


def kmeans_fit(x, init, n_iter: int, weights=None, centroids=None, labels=None, counts=None,
               objective=None, ws=None, assign_events=None):
    """n_iter Lloyd iterations from init.  Returns (centroids, labels, counts,
    objective [B, n_iter] float64).  assign_events: None, or 2 * n_iter
    recorded torch.cuda.Event objects (enable_timing=True) of the tensors'
    device; event 2t is re-recorded right before iteration t's assignment
    kernels and event 2t + 1 right after them (kmeans_fit_timed)."""
    B, N, d = _points(x)
    _dev_tensor(init, "init", torch.float32)
    if init.dim() != 3 or init.shape[0] != B or init.shape[2] != d:
        raise ValueError("init must be [B, K, d] float32")
    K = init.shape[1]
    dev = x.device
    if weights is not None:
        _dev_tensor(weights, "weights", torch.float32, (B, N))
    centroids = torch.empty_like(init) if centroids is None else \
        _dev_tensor(centroids, "centroids", torch.float32, init.shape)
    labels = torch.empty((B, N), dtype=torch.int32, device=dev) if labels is None else \
        _dev_tensor(labels, "labels", torch.int32, (B, N))
    counts = torch.empty((B, K), dtype=torch.int32, device=dev) if counts is None else \
        _dev_tensor(counts, "counts", torch.int32, (B, K))
    objective = torch.empty((B, max(n_iter, 0)), dtype=torch.float64, device=dev) if objective is None else \
        _dev_tensor(objective, "objective", torch.float64, (B, n_iter))
    ws = _ws(ws, B, N, d, K, x.dtype, dev)
    if assign_events is None:
        st = _lib.load().kmeans_fit(_ptr(x), _DT[x.dtype], _ptr(weights), B, N, d, K, _ptr(init), int(n_iter),
                                    _ptr(centroids), _ptr(labels), _ptr(counts), _ptr(objective), _ptr(ws),
                                    ws.numel(), _stream(dev))
        _lib.check(st, "kmeans_fit")
        return centroids, labels, counts, objective
    if len(assign_events) != 2 * n_iter:
        raise ValueError(f"assign_events must hold 2 * n_iter = {2 * n_iter} events")
    handles = []
    for e in assign_events:
        h = getattr(e, "cuda_event", 0)
        if not h:
            raise ValueError("assign_events must be torch.cuda.Event objects recorded once (so that they exist)")
        handles.append(h)
    arr = (ctypes.c_void_p * len(handles))(*handles)
    st = _lib.load().kmeans_fit_timed(_ptr(x), _DT[x.dtype], _ptr(weights), B, N, d, K, _ptr(init), int(n_iter),
                                      _ptr(centroids), _ptr(labels), _ptr(counts), _ptr(objective), arr, _ptr(ws),
                                      ws.numel(), _stream(dev))
    _lib.check(st, "kmeans_fit_timed")
    return centroids, labels, counts, objective


def kmeans_fit_static(x, init, n_iter: int, weights=None, centroids=None, labels=None, counts=None,
                      objective=None):
    """kmeans_fit without a workspace: the library's static per-device scratch
    (kmeans_fit_static_max_bytes() bytes) serves instead, so the call
    allocates nothing itself (pass every output tensor to allocate nothing
    here either).  Returns (centroids, labels, counts, objective)."""
    B, N, d = _points(x)
    _dev_tensor(init, "init", torch.float32)
    if init.dim() != 3 or init.shape[0] != B or init.shape[2] != d:
        raise ValueError("init must be [B, K, d] float32")
    K = init.shape[1]
    dev = x.device
    if weights is not None:
        _dev_tensor(weights, "weights", torch.float32, (B, N))
    centroids = torch.empty_like(init) if centroids is None else \
        _dev_tensor(centroids, "centroids", torch.float32, init.shape)
    labels = torch.empty((B, N), dtype=torch.int32, device=dev) if labels is None else \
        _dev_tensor(labels, "labels", torch.int32, (B, N))
    counts = torch.empty((B, K), dtype=torch.int32, device=dev) if counts is None else \
        _dev_tensor(counts, "counts", torch.int32, (B, K))
    objective = torch.empty((B, max(n_iter, 0)), dtype=torch.float64, device=dev) if objective is None else \
        _dev_tensor(objective, "objective", torch.float64, (B, n_iter))
    st = _lib.load().kmeans_fit_static(_ptr(x), _DT[x.dtype], _ptr(weights), B, N, d, K, _ptr(init), int(n_iter),
                                       _ptr(centroids), _ptr(labels), _ptr(counts), _ptr(objective), _stream(dev))
    _lib.check(st, "kmeans_fit_static")
    return centroids, labels, counts, objective


def kmeans_optimal_1d(x, K: int, weights=None, centroids=None, labels=None, counts=None, objective=None, ws=None):
    """Globally optimal weighted 1D k-means of every row of x [B, N] (or
    [B, N, 1]).  Returns (centroids [B, K] float32 ascending, labels [B, N]
    int32, counts [B, K] int32, objective [B] float64)."""
    _dev_tensor(x, "x")
    if x.dim() == 3 and x.shape[2] == 1:
        B, N = x.shape[0], x.shape[1]
    elif x.dim() == 2:
        B, N = x.shape
    else:
        raise ValueError("x must be [B, N] or [B, N, 1]")
    if x.dtype not in _DT:
        raise TypeError(f"x dtype {x.dtype} is not float32 / float16 / bfloat16")
    dev = x.device
    if weights is not None:
        _dev_tensor(weights, "weights", torch.float32, (B, N))
    centroids = torch.empty((B, K), dtype=torch.float32, device=dev) if centroids is None else \
        _dev_tensor(centroids, "centroids", torch.float32, (B, K))
    labels = torch.empty((B, N), dtype=torch.int32, device=dev) if labels is None else \
        _dev_tensor(labels, "labels", torch.int32, (B, N))
    counts = torch.empty((B, K), dtype=torch.int32, device=dev) if counts is None else \
        _dev_tensor(counts, "counts", torch.int32, (B, K))
    objective = torch.empty((B,), dtype=torch.float64, device=dev) if objective is None else \
        _dev_tensor(objective, "objective", torch.float64, (B,))
    L = _lib.load()
    if ws is None:
        n = L.kmeans_optimal_1d_workspace_bytes(B, N, K)
        ws = torch.empty(max(int(n), 256), dtype=torch.uint8, device=dev)
    _dev_tensor(ws, "workspace", torch.uint8)
    st = L.kmeans_optimal_1d(_ptr(x), _DT[x.dtype], _ptr(weights), B, N, K, _ptr(centroids), _ptr(labels),
                             _ptr(counts), _ptr(objective), _ptr(ws), ws.numel(), _stream(dev))
    _lib.check(st, "kmeans_optimal_1d")
    return centroids, labels, counts, objective


def kmeans_fit_stream(x_host, init, n_iter: int, weights=None, chunk: int = 1 << 22, centroids=None, labels=None,
                      counts=None, objective=None, ws=None):
    """n_iter Lloyd iterations of one problem whose points x_host [N, d] (or
    [1, N, d]) stay in host memory (a CPU tensor, ideally pinned), streamed
    to the GPU in chunks of `chunk` points.  init [K, d] (or [1, K, d])
    float32 on the GPU.  Returns (centroids [K, d], labels [N] (None unless
    True or a tensor is passed), counts [K], objective [n_iter] float64)."""
    if not isinstance(x_host, torch.Tensor) or x_host.is_cuda:
        raise ValueError("x_host must be a CPU tensor")
    if not x_host.is_contiguous():
        raise ValueError("x_host must be contiguous")
    if x_host.dim() == 3 and x_host.shape[0] == 1:
        x_host = x_host[0]
    if x_host.dim() != 2:
        raise ValueError("x_host must be [N, d]")
    if x_host.dtype not in _DT:
        raise TypeError(f"x dtype {x_host.dtype} is not float32 / float16 / bfloat16")
    N, d = x_host.shape
    _dev_tensor(init, "init", torch.float32)
    if init.dim() == 3 and init.shape[0] == 1:
        init = init[0]
    if init.dim() != 2 or init.shape[1] != d:
        raise ValueError("init must be [K, d] float32")
    K = init.shape[0]
    dev = init.device
    if weights is not None:
        if not isinstance(weights, torch.Tensor) or weights.is_cuda or weights.dtype != torch.float32 \
                or tuple(weights.shape) != (N,) or not weights.is_contiguous():
            raise ValueError("weights must be a contiguous float32 CPU tensor [N]")
    centroids = torch.empty_like(init) if centroids is None else \
        _dev_tensor(centroids, "centroids", torch.float32, init.shape)
    if labels is True:
        labels = torch.empty((N,), dtype=torch.int32, device=dev)
    elif labels is not None:
        _dev_tensor(labels, "labels", torch.int32, (N,))
    counts = torch.empty((K,), dtype=torch.int32, device=dev) if counts is None else \
        _dev_tensor(counts, "counts", torch.int32, (K,))
    objective = torch.empty((max(n_iter, 0),), dtype=torch.float64, device=dev) if objective is None else \
        _dev_tensor(objective, "objective", torch.float64, (n_iter,))
    L = _lib.load()
    if ws is None:
        # 0 for arguments the entry point rejects: it then reports why
        n = L.kmeans_stream_workspace_bytes(N, d, K, _DT[x_host.dtype], chunk)
        ws = torch.empty(max(int(n), 256), dtype=torch.uint8, device=dev)
    _dev_tensor(ws, "workspace", torch.uint8)
    st = L.kmeans_fit_stream(_ptr(x_host), _DT[x_host.dtype], _ptr(weights), N, d, K, _ptr(init), int(n_iter),
                             _ptr(centroids), _ptr(labels), _ptr(counts), _ptr(objective), int(chunk), _ptr(ws),
                             ws.numel(), _stream(dev))
    _lib.check(st, "kmeans_fit_stream")
    return centroids, labels, counts, objective


def emeans_steps(N: int, batch: int, epochs: int) -> int:
    """Number of e-means steps: epochs times the batches of one pass."""
    return epochs * ((N + batch - 1) // batch) if N > 0 else 0


def kmeans_emeans(x, init, batch: int, epochs: int, alpha0: float, floor_frac: float = 0.1, dead_frac: float = 0.0,
                  eps: float = 1e-3, uniforms=None, centroids=None, labels=None, counts=None, objective=None,
                  ws=None):
    """e-means (moving-average mini-batch k-means) of one problem x [N, d]
    (or [1, N, d]) on the GPU from init [K, d] float32.  uniforms [T, K]
    float32 on the GPU (T = emeans_steps(N, batch, epochs)) are the split
    draws, needed when dead_frac > 0.  Returns (centroids [K, d], labels [N]
    (None unless True or a tensor is passed), counts [K], objective [T]
    float64)."""
    _dev_tensor(x, "x")
    if x.dim() == 3 and x.shape[0] == 1:
        x = x[0]
    if x.dim() != 2:
        raise ValueError("x must be [N, d]")
    if x.dtype not in _DT:
        raise TypeError(f"x dtype {x.dtype} is not float32 / float16 / bfloat16")
    N, d = x.shape
    _dev_tensor(init, "init", torch.float32)
    if init.dim() == 3 and init.shape[0] == 1:
        init = init[0]
    if init.dim() != 2 or init.shape[1] != d:
        raise ValueError("init must be [K, d] float32")
    K = init.shape[0]
    dev = x.device
    T = emeans_steps(N, batch, epochs) if batch >= 1 and epochs >= 1 else 0
    if uniforms is not None:
        _dev_tensor(uniforms, "uniforms", torch.float32, (T, K))
    centroids = torch.empty_like(init) if centroids is None else \
        _dev_tensor(centroids, "centroids", torch.float32, init.shape)
    if labels is True:
        labels = torch.empty((N,), dtype=torch.int32, device=dev)
    elif labels is not None:
        _dev_tensor(labels, "labels", torch.int32, (N,))
    counts = torch.empty((K,), dtype=torch.int32, device=dev) if counts is None else \
        _dev_tensor(counts, "counts", torch.int32, (K,))
    objective = torch.empty((T,), dtype=torch.float64, device=dev) if objective is None else \
        _dev_tensor(objective, "objective", torch.float64, (T,))
    L = _lib.load()
    if ws is None:
        # 0 for arguments the entry point rejects: it then reports why
        n = L.kmeans_emeans_workspace_bytes(N, d, K, _DT[x.dtype], int(batch))
        ws = torch.empty(max(int(n), 256), dtype=torch.uint8, device=dev)
    _dev_tensor(ws, "workspace", torch.uint8)
    st = L.kmeans_emeans(_ptr(x), _DT[x.dtype], N, d, K, _ptr(init), int(batch), int(epochs), float(alpha0),
                         float(floor_frac), float(dead_frac), float(eps), _ptr(uniforms), _ptr(centroids),
                         _ptr(labels), _ptr(counts), _ptr(objective), _ptr(ws), ws.numel(), _stream(dev))
    _lib.check(st, "kmeans_emeans")
    return centroids, labels, counts, objective
