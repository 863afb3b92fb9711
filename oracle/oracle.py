"""ctypes wrapper of the C oracle (plain Lloyd k-means in fp64).

TEST INFRASTRUCTURE ONLY.  Imported by the tests, the smoke check and the
benchmark's CPU-baseline leg; never by the library.  It shares no code with
the GPU path: the only common module is the seeded input generator.

Arrays are numpy.  Points are passed as their stored bits: float32 arrays for
fp32, uint16 arrays for fp16 / bf16 (with the dtype name), and are decoded to
fp64 exactly inside the C code.
"""
from __future__ import annotations

import contextlib
import ctypes as C
import os

import numpy as np

from . import build as _build

DTYPES = {"f32": 0, "f16": 1, "bf16": 2}

_lib = None


def load_library(path: str):
    """A ctypes handle of an oracle library built from this file's C source
    (the tests also load deliberately broken copies to check the pins)."""
    L = C.CDLL(path)
    p = C.c_void_p
    i64 = C.c_int64
    L.oracle_decode_one.argtypes = [C.c_uint32, C.c_int]
    L.oracle_decode_one.restype = C.c_double
    L.oracle_round_one.argtypes = [C.c_float, C.c_int]
    L.oracle_round_one.restype = C.c_uint32
    L.oracle_decode.argtypes = [p, C.c_int, i64, p]
    L.oracle_round.argtypes = [p, i64, C.c_int, p]
    L.oracle_assign.argtypes = [p, i64, i64, i64, p, i64, p, p, p]
    L.oracle_update.argtypes = [p, p, p, i64, i64, i64, i64, p, p, p, p, p]
    L.oracle_objective.argtypes = [p, p, p, i64, i64, i64, p, i64, p]
    L.oracle_update_bits.argtypes = [p, C.c_int, p, p, i64, i64, i64, i64, p, p, p, p, p]
    L.oracle_update_bits.restype = C.c_int
    L.oracle_objective_bits.argtypes = [p, C.c_int, p, p, i64, i64, i64, p, i64, p]
    L.oracle_objective_bits.restype = C.c_int
    L.oracle_fit.argtypes = [p, C.c_int, p, i64, i64, i64, i64, p, C.c_int32,
                             p, p, p, p, p, p]
    L.oracle_fit.restype = C.c_int
    L.oracle_num_threads.restype = C.c_int
    L.oracle_optimal_1d.argtypes = [p, p, i64, i64, i64, p, p, p, p]
    L.oracle_optimal_1d.restype = C.c_int
    L.oracle_emeans.argtypes = [p, C.c_int, i64, i64, i64, p, i64, C.c_int32, C.c_double, C.c_double, C.c_double,
                                C.c_double, p, p, p, p, p]
    L.oracle_emeans.restype = C.c_int
    return L


def lib():
    """The loaded oracle library; compiled first if it has not been built."""
    global _lib
    if _lib is None:
        path = os.environ.get("KM_ORACLE_LIBRARY") or _build.LIB
        if not os.path.exists(path):
            _build.build()
        _lib = load_library(path)
    return _lib


@contextlib.contextmanager
def using_library(path: str):
    """Route every call of this module to another build of the oracle source
    for the duration of the block."""
    global _lib
    saved = lib()
    _lib = load_library(path)
    try:
        yield
    finally:
        _lib = saved


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().oracle_num_threads())


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 values of stored elements (float32, or uint16 bits of fp16/bf16)."""
    want = np.float32 if dtype == "f32" else np.uint16
    bits = np.ascontiguousarray(bits, dtype=want)
    out = np.empty(bits.shape, dtype=np.float64)
    lib().oracle_decode(_ptr(bits), DTYPES[dtype], bits.size, _ptr(out))
    return out


def round_to(c: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> stored bits of dtype with IEEE round-to-nearest-even."""
    c = np.ascontiguousarray(c, dtype=np.float32)
    out = np.empty(c.shape, dtype=np.float32 if dtype == "f32" else np.uint16)
    lib().oracle_round(_ptr(c), c.size, DTYPES[dtype], _ptr(out))
    return out


def assign(X: np.ndarray, Chat: np.ndarray):
    """Assignment stage.  X [B,N,d] fp64, Chat [B,K,d] fp64 (already in the
    point dtype's values).  Returns labels int32 [B,N], d1 (nearest squared
    distance) and d2 (second nearest; inf when K == 1), fp64 [B,N]."""
    X = np.ascontiguousarray(X, dtype=np.float64)
    Chat = np.ascontiguousarray(Chat, dtype=np.float64)
    B, N, d = X.shape
    K = Chat.shape[1]
    assert Chat.shape == (B, K, d)
    labels = np.empty((B, N), np.int32)
    d1 = np.empty((B, N), np.float64)
    d2 = np.empty((B, N), np.float64)
    lib().oracle_assign(_ptr(X), B, N, d, _ptr(Chat), K, _ptr(labels), _ptr(d1), _ptr(d2))
    return labels, d1, d2


def update(X: np.ndarray, w, labels: np.ndarray, c_old: np.ndarray):
    """Update stage.  X [B,N,d] fp64, w [B,N] (or None), labels int32 [B,N],
    c_old [B,K,d] fp32.  Returns (c_new fp32, counts int32 [B,K],
    S fp64 [B,K,d], W fp64 [B,K])."""
    X = np.ascontiguousarray(X, dtype=np.float64)
    B, N, d = X.shape
    c_old = np.ascontiguousarray(c_old, dtype=np.float32)
    K = c_old.shape[1]
    labels = np.ascontiguousarray(labels, dtype=np.int32)
    assert labels.shape == (B, N)
    if labels.size and (labels.min() < 0 or labels.max() >= K):
        raise ValueError("label out of range")
    wd = None if w is None else np.ascontiguousarray(w, dtype=np.float64)
    c_new = np.empty_like(c_old)
    counts = np.empty((B, K), np.int32)
    S = np.empty((B, K, d), np.float64)
    W = np.empty((B, K), np.float64)
    lib().oracle_update(_ptr(X), _ptr(wd), _ptr(labels), B, N, d, K, _ptr(c_old),
                        _ptr(c_new), _ptr(counts), _ptr(S), _ptr(W))
    return c_new, counts, S, W


def objective(X: np.ndarray, w, labels: np.ndarray, Chat: np.ndarray) -> np.ndarray:
    """J [B] = sum_i w_i |x_i - c_{l_i}|^2 of given labels (fp64)."""
    X = np.ascontiguousarray(X, dtype=np.float64)
    B, N, d = X.shape
    Chat = np.ascontiguousarray(Chat, dtype=np.float64)
    K = Chat.shape[1]
    labels = np.ascontiguousarray(labels, dtype=np.int32)
    wd = None if w is None else np.ascontiguousarray(w, dtype=np.float64)
    J = np.empty(B, np.float64)
    lib().oracle_objective(_ptr(X), _ptr(wd), _ptr(labels), B, N, d, _ptr(Chat), K, _ptr(J))
    return J


def _bits(x_bits: np.ndarray, dtype: str) -> np.ndarray:
    want = np.float32 if dtype == "f32" else np.uint16
    if x_bits.dtype != want:
        raise TypeError(f"stored bits of {dtype} must be {np.dtype(want).name}")
    return np.ascontiguousarray(x_bits)


def update_bits(x_bits: np.ndarray, dtype: str, w, labels: np.ndarray, c_old: np.ndarray):
    """The update stage of `update`, reading the points as stored bits
    x_bits [B,N,d] (float32, or uint16 for fp16 / bf16) instead of decoded
    fp64 (same arithmetic, same order, same results).  w [B,N] float32 or
    None.  Returns (c_new fp32, counts int32 [B,K], S fp64, W fp64)."""
    x_bits = _bits(x_bits, dtype)
    B, N, d = x_bits.shape
    c_old = np.ascontiguousarray(c_old, dtype=np.float32)
    K = c_old.shape[1]
    assert c_old.shape == (B, K, d)
    labels = np.ascontiguousarray(labels, dtype=np.int32)
    assert labels.shape == (B, N)
    w32 = None if w is None else np.ascontiguousarray(w, dtype=np.float32)
    c_new = np.empty_like(c_old)
    counts = np.empty((B, K), np.int32)
    S = np.empty((B, K, d), np.float64)
    W = np.empty((B, K), np.float64)
    rc = lib().oracle_update_bits(_ptr(x_bits), DTYPES[dtype], _ptr(w32), _ptr(labels), B, N, d, K, _ptr(c_old),
                                  _ptr(c_new), _ptr(counts), _ptr(S), _ptr(W))
    if rc != 0:
        raise ValueError("oracle_update_bits: label out of range, or out of host memory")
    return c_new, counts, S, W


def objective_bits(x_bits: np.ndarray, dtype: str, w, labels: np.ndarray, Chat: np.ndarray) -> np.ndarray:
    """`objective` of given labels, reading the points as stored bits
    (same terms, added in the same order)."""
    x_bits = _bits(x_bits, dtype)
    B, N, d = x_bits.shape
    Chat = np.ascontiguousarray(Chat, dtype=np.float64)
    K = Chat.shape[1]
    labels = np.ascontiguousarray(labels, dtype=np.int32)
    w32 = None if w is None else np.ascontiguousarray(w, dtype=np.float32)
    J = np.empty(B, np.float64)
    rc = lib().oracle_objective_bits(_ptr(x_bits), DTYPES[dtype], _ptr(w32), _ptr(labels), B, N, d, _ptr(Chat), K,
                                     _ptr(J))
    if rc != 0:
        raise MemoryError("oracle_objective_bits ran out of host memory")
    return J


def fit(x_bits: np.ndarray, dtype: str, w, init: np.ndarray, n_iter: int) -> dict:
    """n_iter Lloyd iterations.  x_bits [B,N,d] stored bits, w [B,N] fp32 or
    None, init [B,K,d] fp32.  Returns centroids, labels and d1/d2 of the last
    assignment, counts of the last update, and J [B, n_iter]."""
    want = np.float32 if dtype == "f32" else np.uint16
    x_bits = np.ascontiguousarray(x_bits, dtype=want)
    B, N, d = x_bits.shape
    init = np.ascontiguousarray(init, dtype=np.float32)
    K = init.shape[1]
    assert init.shape == (B, K, d)
    w32 = None if w is None else np.ascontiguousarray(w, dtype=np.float32)
    C_out = np.empty_like(init)
    labels = np.empty((B, N), np.int32)
    counts = np.empty((B, K), np.int32)
    J = np.empty((B, n_iter), np.float64)
    d1 = np.empty((B, N), np.float64)
    d2 = np.empty((B, N), np.float64)
    rc = lib().oracle_fit(_ptr(x_bits), DTYPES[dtype], _ptr(w32), B, N, d, K, _ptr(init),
                          int(n_iter), _ptr(C_out), _ptr(labels), _ptr(counts), _ptr(J),
                          _ptr(d1), _ptr(d2))
    if rc != 0:
        raise MemoryError("oracle_fit ran out of host memory")
    return dict(centroids=C_out, labels=labels, counts=counts, J=J, d1=d1, d2=d2)


def optimal_1d(X: np.ndarray, w, K: int) -> dict:
    """Globally optimal weighted 1D k-means of every row.  X [B,N] fp64 (or
    [B,N,1]), w [B,N] or None, 1 <= K <= N.  Returns J [B] (fp64), means
    [B,K] (fp64, ascending), labels int32 [B,N] (run index of every point)
    and counts int32 [B,K]."""
    X = np.ascontiguousarray(X, dtype=np.float64)
    if X.ndim == 3:
        assert X.shape[2] == 1
        X = X[..., 0]
    X = np.ascontiguousarray(X)
    B, N = X.shape
    wd = None if w is None else np.ascontiguousarray(w, dtype=np.float64)
    J = np.empty(B, np.float64)
    means = np.empty((B, K), np.float64)
    labels = np.empty((B, N), np.int32)
    counts = np.empty((B, K), np.int32)
    rc = lib().oracle_optimal_1d(_ptr(X), _ptr(wd), B, N, int(K), _ptr(J), _ptr(means), _ptr(labels),
                                 _ptr(counts))
    if rc != 0:
        raise ValueError(f"oracle_optimal_1d failed (K={K}, N={N}, or out of memory)")
    return dict(J=J, means=means, labels=labels, counts=counts)


def emeans(x_bits: np.ndarray, dtype: str, init: np.ndarray, batch: int, epochs: int, alpha0: float,
           floor_frac: float, dead_frac: float, eps: float, uniforms: np.ndarray) -> dict:
    """e-means on one problem.  x_bits [N, d] (or [1, N, d]) stored bits, init
    [K, d] float32, uniforms [T * K] float32 in [0, 1) with T = epochs *
    ceil(N / batch).  Returns centroids [K, d] float32, J [T] (each batch's
    assignment cost), labels int32 [N] and counts int32 [K] of the last
    epoch."""
    want = np.float32 if dtype == "f32" else np.uint16
    x_bits = np.ascontiguousarray(x_bits, dtype=want)
    if x_bits.ndim == 3:
        x_bits = x_bits[0]
    N, d = x_bits.shape
    init = np.ascontiguousarray(init, dtype=np.float32).reshape(-1, d)
    K = init.shape[0]
    T = epochs * ((N + batch - 1) // batch)
    uniforms = np.ascontiguousarray(uniforms, dtype=np.float32).reshape(-1)
    assert uniforms.size == T * K
    C_out = np.empty_like(init)
    J = np.empty(T, np.float64)
    labels = np.empty(N, np.int32)
    counts = np.empty(K, np.int32)
    rc = lib().oracle_emeans(_ptr(x_bits), DTYPES[dtype], N, d, K, _ptr(init), int(batch), int(epochs),
                             float(alpha0), float(floor_frac), float(dead_frac), float(eps), _ptr(uniforms),
                             _ptr(C_out), _ptr(J), _ptr(labels), _ptr(counts))
    if rc != 0:
        raise ValueError("oracle_emeans failed (arguments out of range, or out of memory)")
    return dict(centroids=C_out, J=J, labels=labels, counts=counts)


def near_tie(d1: np.ndarray, d2: np.ndarray, rel: float = 1e-4) -> np.ndarray:
    """Points whose top-2 gap is at most rel * nearest distance.

    d1 == d2 (duplicate centroids, including both zero) is a near tie;
    d1 == 0 < d2 is not; with one centroid (d2 = inf) nothing is."""
    return (d2 - d1) <= rel * d1
