"""The C ABI library on a machine without a GPU: it loads, exports every
symbol the header declares, and rejects invalid arguments on the host before
any HIP call."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    from exact_lloyd_means_03_amd import _lib
    return _lib.load()


def _header_functions():
    text = open(os.path.join(ROOT, "include", "kmeans.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kmeans_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    from exact_lloyd_means_03_amd import _lib
    names = _header_functions()
    assert names == sorted(_lib.SIGNATURES)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    assert lib.kmeans_status_str(0) == b"ok"
    assert lib.kmeans_status_str(3) == b"workspace too small"
    assert lib.kmeans_version() >= 100


def test_workspace_bytes(lib):
    n = lib.kmeans_workspace_bytes(1, 1 << 20, 128, 8192, 1)
    # at least labels, perm, sums and the padded fp16 centroids
    assert n >= (1 << 20) * 8 + 8192 * 128 * 4 + 8192 * 128 * 2
    assert n % 256 == 0
    assert lib.kmeans_workspace_bytes(1, 100, 0, 4, 1) == 0       # d < 1
    assert lib.kmeans_workspace_bytes(1, 100, 513, 4, 1) == 0     # d > 512
    assert lib.kmeans_workspace_bytes(1, 100, 300, 4, 0) == 0     # float32 rows above 256
    assert lib.kmeans_workspace_bytes(1, 100, 512, 4, 2) > 0
    assert lib.kmeans_workspace_bytes(1, 100, 8, 40000, 1) == 0   # K > 32768
    assert lib.kmeans_workspace_bytes(-1, 100, 8, 4, 1) == 0
    assert lib.kmeans_workspace_bytes(1, 100, 8, 4, 7) == 0       # dtype


FAKE = C.c_void_p(0x1000)  # never dereferenced: every case fails before any HIP call


@pytest.mark.parametrize("args,status", [
    # x NULL
    (dict(x=None), 1),
    # K = 0
    (dict(K=0), 1),
    # d above the limits: 512 for 16-bit points, 256 for float32 points
    (dict(d=513), 2),
    (dict(d=300, xt=0), 2),
    # unsupported dtype
    (dict(xt=5), 2),
    # workspace too small
    (dict(ws_bytes=16), 3),
    # misaligned workspace
    (dict(ws=C.c_void_p(0x1008)), 1),
    # negative N
    (dict(N=-3), 1),
])
def test_assign_rejects(lib, args, status):
    a = dict(x=FAKE, xt=1, B=1, N=100, d=8, C=FAKE, K=4, w=None, labels=FAKE, md=None, obj=None,
             ws=C.c_void_p(0x100000), ws_bytes=1 << 30, stream=None)
    a.update(args)
    st = lib.kmeans_assign(a["x"], a["xt"], a["B"], a["N"], a["d"], a["C"], a["K"], a["w"], a["labels"],
                           a["md"], a["obj"], a["ws"], a["ws_bytes"], a["stream"])
    assert st == status
    assert lib.kmeans_last_error() != b""


def test_update_and_fit_reject(lib):
    ws = C.c_void_p(0x100000)
    assert lib.kmeans_update(FAKE, 1, None, 1, 10, 8, None, 4, FAKE, FAKE, None, ws, 1 << 30, None) == 1
    assert lib.kmeans_update(FAKE, 1, None, 1, 10, 8, FAKE, 40000, FAKE, FAKE, None, ws, 1 << 30, None) == 2
    assert lib.kmeans_fit(FAKE, 1, None, 1, 10, 8, 4, FAKE, -1, FAKE, None, None, None, ws, 1 << 30, None) == 1
    assert lib.kmeans_fit(FAKE, 2, None, 1, 10, 8, 4, FAKE, 3, FAKE, None, None, None, ws, 100, None) == 3
    assert lib.kmeans_sort_labels(None, 1, 10, 4, None, None, None, ws, 1 << 30, None) == 1
    assert b"labels" in lib.kmeans_last_error()
    # B*N*d beyond the 64-bit guard
    assert lib.kmeans_fit(FAKE, 1, None, 65535, 0x7fffffff, 256, 4, FAKE, 1, FAKE, None, None, None,
                          ws, 1 << 62, None) == 2


def test_python_binding_requires_gpu_tensors():
    import torch
    import exact_lloyd_means_03_amd as km
    x = torch.zeros(1, 10, 8)
    with pytest.raises(ValueError, match="GPU"):
        km.kmeans_assign(x, torch.zeros(1, 4, 8))


def test_optimal_1d_rejects(lib):
    ws = C.c_void_p(0x100000)
    n = lib.kmeans_optimal_1d_workspace_bytes(4096, 4096, 16)
    # D per row, the cuts of every layer (uint16) and the sort permutation
    assert n >= 4096 * (4097 * 8 + 16 * 4097 * 2 + 4096 * 4) and n % 256 == 0
    assert lib.kmeans_optimal_1d_workspace_bytes(1, 4097, 16) == 0   # N above the limit
    assert lib.kmeans_optimal_1d_workspace_bytes(1, 10, 11) == 0     # K > N
    assert lib.kmeans_optimal_1d_workspace_bytes(1, 4000, 257) == 0  # K above the limit

    def call(**kw):
        a = dict(x=FAKE, xt=0, w=None, B=2, N=100, K=4, C=FAKE, ws=ws, ws_bytes=1 << 30)
        a.update(kw)
        return lib.kmeans_optimal_1d(a["x"], a["xt"], a["w"], a["B"], a["N"], a["K"], a["C"], None, None, None,
                                     a["ws"], a["ws_bytes"], None)

    assert call(K=0) == 1
    assert call(K=101) == 1 and b"K <= N" in lib.kmeans_last_error()
    assert call(N=5000, K=4) == 2
    assert call(N=1000, K=300) == 2
    assert call(xt=9) == 2
    assert call(x=None) == 1
    assert call(C=None) == 1
    assert call(ws_bytes=100) == 3
    assert call(ws=C.c_void_p(0x100010)) == 1
    assert call(N=-1) == 1


def test_fit_stream_rejects(lib):
    ws = C.c_void_p(0x100000)
    assert lib.kmeans_stream_workspace_bytes(1 << 20, 128, 4096, 1, 1 << 18) > 0
    assert lib.kmeans_stream_workspace_bytes(1000, 1, 4, 1, 4096) == 0      # d = 1
    assert lib.kmeans_stream_workspace_bytes(1000, 16, 4, 1, 0) == 0        # chunk < 1

    def call(**kw):
        a = dict(x=FAKE, xt=1, w=None, N=1000, d=16, K=4, init=FAKE, n_iter=2, C=FAKE, chunk=4096, ws=ws,
                 ws_bytes=1 << 30)
        a.update(kw)
        return lib.kmeans_fit_stream(a["x"], a["xt"], a["w"], a["N"], a["d"], a["K"], a["init"], a["n_iter"],
                                     a["C"], None, None, None, a["chunk"], a["ws"], a["ws_bytes"], None)

    assert call(d=1) == 2 and b"d >= 2" in lib.kmeans_last_error()
    assert call(chunk=0) == 1
    assert call(n_iter=-1) == 1
    assert call(x=None) == 1
    assert call(init=None) == 1
    assert call(ws_bytes=64) == 3
    assert call(K=0) == 1
    assert call(xt=4) == 2


def test_emeans_rejects(lib):
    ws = C.c_void_p(0x100000)
    n = lib.kmeans_emeans_workspace_bytes(1 << 20, 96, 16384, 2, 65536)
    # the float64 sums S and last-epoch sums F, and the batch's labels and permutation
    assert n >= 2 * 16384 * 96 * 8 + 2 * 65536 * 4 and n % 256 == 0
    assert lib.kmeans_emeans_workspace_bytes(1000, 16, 4, 1, 0) == 0       # batch < 1
    assert lib.kmeans_emeans_workspace_bytes(1000, 1, 20000, 0, 64) == 0   # d = 1 and K > 16384
    assert lib.kmeans_emeans_workspace_bytes(1000, 16, 40000, 1, 64) == 0  # K > 32768

    def call(**kw):
        a = dict(x=FAKE, xt=1, N=1000, d=16, K=4, init=FAKE, batch=100, epochs=2, alpha0=0.5, floor=0.1,
                 dead=0.0, eps=1e-3, u=None, C=FAKE, ws=ws, ws_bytes=1 << 30)
        a.update(kw)
        return lib.kmeans_emeans(a["x"], a["xt"], a["N"], a["d"], a["K"], a["init"], a["batch"], a["epochs"],
                                 a["alpha0"], a["floor"], a["dead"], a["eps"], a["u"], a["C"], None, None, None,
                                 a["ws"], a["ws_bytes"], None)

    assert call(batch=0) == 1 and b"batch" in lib.kmeans_last_error()
    assert call(epochs=0) == 1
    assert call(alpha0=0.0) == 1 and b"alpha0" in lib.kmeans_last_error()
    assert call(alpha0=1.5) == 1
    assert call(floor=-0.1) == 1
    assert call(floor=float("nan")) == 1
    assert call(dead=-1.0) == 1
    assert call(eps=1.0) == 1
    assert call(dead=0.5) == 1 and b"uniforms" in lib.kmeans_last_error()  # splits need the draws
    assert call(x=None) == 1
    assert call(init=None) == 1
    assert call(C=None) == 1
    assert call(K=0) == 1
    assert call(K=40000) == 2
    assert call(d=1, K=20000, xt=0) == 2
    assert call(xt=5) == 2
    assert call(ws_bytes=64) == 3
    assert call(ws=C.c_void_p(0x100010)) == 1


def test_fit_static_rejects_before_any_hip_call(lib):
    # the static scratch is 64 MiB per device; shapes that need more are
    # refused on the host, as are invalid arguments
    assert lib.kmeans_fit_static_max_bytes() == 64 << 20

    def call(**kw):
        a = dict(x=FAKE, xt=1, B=1, N=1 << 24, d=128, K=4096, init=FAKE, n_iter=2, C=FAKE)
        a.update(kw)
        return lib.kmeans_fit_static(a["x"], a["xt"], None, a["B"], a["N"], a["d"], a["K"], a["init"], a["n_iter"],
                                     a["C"], None, None, None, None)

    assert lib.kmeans_workspace_bytes(1, 1 << 24, 128, 4096, 1) > lib.kmeans_fit_static_max_bytes()
    assert call() == 3 and b"static" in lib.kmeans_last_error()
    assert call(x=None) == 1
    assert call(init=None) == 1
    assert call(C=None) == 1
    assert call(n_iter=-1) == 1
    assert call(K=0) == 1
    assert call(xt=7) == 2
    assert call(d=1, K=20000, xt=0) == 2


def test_fit_timed_rejects(lib):
    ws = C.c_void_p(0x100000)
    ev = (C.c_void_p * 4)(0x10, 0x20, 0x30, 0x40)
    call = lambda events, n_iter=2, ws_bytes=1 << 30: lib.kmeans_fit_timed(  # noqa: E731
        FAKE, 1, None, 1, 10, 8, 4, FAKE, n_iter, FAKE, None, None, None, events, ws, ws_bytes, None)
    assert call(None) == 1 and b"assign_events" in lib.kmeans_last_error()
    bad = (C.c_void_p * 4)(0x10, 0x20, None, 0x40)
    assert call(bad) == 1 and b"assign_events[2]" in lib.kmeans_last_error()
    assert call(ev, n_iter=-1) == 1
    assert call(ev, ws_bytes=16) == 3
