"""ctypes declarations of the C ABI in include/kmeans.h.

The library is loaded from this package's directory.  There is no fallback:
if libkmeans_mi355x.so is missing, loading raises, so nothing can silently
run a different implementation.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# KM_LIBRARY may name another build of the same sources (the sanitized host
# build of the CPU test tier); by default the library next to this file.
LIB_PATH = os.environ.get("KM_LIBRARY") or os.path.join(HERE, "libkmeans_mi355x.so")

KM_F32, KM_F16, KM_BF16 = 0, 1, 2
STATUS = {0: "KM_OK", 1: "KM_EINVAL", 2: "KM_EUNSUPPORTED", 3: "KM_EWORKSPACE", 4: "KM_EHIP"}

# Every symbol the header declares, with (restype, argtypes).
_p, _i64, _i32, _sz = C.c_void_p, C.c_int64, C.c_int32, C.c_size_t
SIGNATURES = {
    "kmeans_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, C.c_int]),
    "kmeans_assign": (C.c_int, [_p, C.c_int, _i64, _i64, _i64, _p, _i64, _p, _p, _p, _p, _p, _sz, _p]),
    "kmeans_sort_labels": (C.c_int, [_p, _i64, _i64, _i64, _p, _p, _p, _p, _sz, _p]),
    "kmeans_update": (C.c_int, [_p, C.c_int, _p, _i64, _i64, _i64, _p, _i64, _p, _p, _p, _p, _sz, _p]),
    "kmeans_fit": (C.c_int, [_p, C.c_int, _p, _i64, _i64, _i64, _i64, _p, _i32, _p, _p, _p, _p, _p, _sz, _p]),
    "kmeans_fit_timed": (C.c_int, [_p, C.c_int, _p, _i64, _i64, _i64, _i64, _p, _i32, _p, _p, _p, _p, _p, _p, _sz,
                                   _p]),
    "kmeans_fit_static_max_bytes": (_sz, []),
    "kmeans_fit_static": (C.c_int, [_p, C.c_int, _p, _i64, _i64, _i64, _i64, _p, _i32, _p, _p, _p, _p, _p]),
    "kmeans_stream_workspace_bytes": (_sz, [_i64, _i64, _i64, C.c_int, _i64]),
    "kmeans_fit_stream": (C.c_int, [_p, C.c_int, _p, _i64, _i64, _i64, _p, _i32, _p, _p, _p, _p, _i64, _p, _sz,
                                    _p]),
    "kmeans_optimal_1d_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "kmeans_optimal_1d": (C.c_int, [_p, C.c_int, _p, _i64, _i64, _i64, _p, _p, _p, _p, _p, _sz, _p]),
    "kmeans_emeans_workspace_bytes": (_sz, [_i64, _i64, _i64, C.c_int, _i64]),
    "kmeans_emeans": (C.c_int, [_p, C.c_int, _i64, _i64, _i64, _p, _i64, _i32, C.c_double, C.c_double, C.c_double,
                                C.c_double, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "kmeans_status_str": (C.c_char_p, [C.c_int]),
    "kmeans_last_error": (C.c_char_p, []),
    "kmeans_version": (C.c_int, []),
}

_lib = None


class KMeansError(RuntimeError):
    """A non-zero km_status returned by the library."""

    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}: {detail}")


def load():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
                "or `python exact_lloyd_means_03_amd/build.py`")
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(status: int, where: str) -> None:
    if status != 0:
        raise KMeansError(status, where, load().kmeans_last_error().decode())
