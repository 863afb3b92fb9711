"""The seeded generators: determinism, shapes and the stated distributions."""
import hashlib

import numpy as np
import torch

import workloads


def _digest(p):
    h = hashlib.sha256()
    h.update(workloads.raw_bits(p.x).tobytes())
    h.update(p.init.numpy().tobytes())
    if p.w is not None:
        h.update(p.w.numpy().tobytes())
    return h.hexdigest()


def test_deterministic_and_seed_sensitive():
    wl = workloads.small("gmm-n1m-k8192-d128-f16", N=5000, K=64, d=16)
    a, b = workloads.generate(wl), workloads.generate(wl)
    assert _digest(a) == _digest(b)
    c = workloads.generate(wl.replace(seed=wl.seed + 1))
    assert _digest(a) != _digest(c)


def test_chunking_does_not_depend_on_threads(monkeypatch):
    wl = workloads.small("gmm-n1m-k8192-d128-f16", N=3 * workloads.CHUNK_ROWS // 2, K=32, d=8)
    a = workloads.generate(wl)
    monkeypatch.setattr(workloads, "_threads", lambda: 1)
    b = workloads.generate(wl)
    assert _digest(a) == _digest(b)


def test_shapes_and_dtypes():
    for name, kw in [("gmm-n8192-k256-d128-f32", {}),
                     ("gmm-b32-n65536-k1024-d128-f16", dict(B=3, N=4096)),
                     ("zipf-n32m-k4096-d128-bf16", dict(N=20000, K=256)),
                     ("rows1d-b4096-n4096-k16-f32", dict(B=5))]:
        wl = workloads.small(name, **kw)
        p = workloads.generate(wl)
        assert p.x.shape == (wl.B, wl.N, wl.d)
        assert p.x.dtype == {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[wl.dtype]
        assert p.init.shape == (wl.B, wl.K, wl.d) and p.init.dtype == torch.float32
        assert (p.w is not None) == wl.weighted


def test_noise_fraction_and_random_init_rows():
    wl = workloads.small("gmm-n1m-k8192-d128-f16", N=20000, K=128, d=32)
    p = workloads.generate(wl)
    x = p.x[0].float().numpy()
    n_noise = int(round(0.05 * wl.N))
    # mixture rows lie within a few sigma of one of the means; uniform noise rows do not
    from scipy.spatial.distance import cdist
    dmin = cdist(x, p.means[0]).min(axis=1)
    assert int((dmin > 0.15 * np.sqrt(wl.d) * 2).sum()) == n_noise
    # random-K init rows are distinct rows of x
    rows = {tuple(r) for r in x}
    init = p.init[0].numpy()
    assert all(tuple(r) in rows for r in init)
    assert len({tuple(r) for r in init}) == wl.K


def test_zipf_head_cluster_share():
    wl = workloads.small("zipf-n32m-k4096-d128-bf16", N=200000, d=4)
    p = workloads.generate(wl)
    # the head component holds p_1 = 1 / sum_k k^-1.2 of the points (~21.5%)
    H = (np.arange(1, 4097, dtype=np.float64) ** -1.2).sum()
    x = p.x[0].float().numpy()
    m0 = p.means[0, 0]
    near = (np.abs(x - m0) < 0.8).all(axis=1).mean()
    assert abs(near - 1 / H) < 0.01


def test_linspace_init_endpoints():
    wl = workloads.small("rows1d-b4096-n4096-k16-f32", B=7)
    p = workloads.generate(wl)
    x = p.x[:, :, 0]
    np.testing.assert_array_equal(p.init[:, 0, 0], x.min(dim=1).values)
    np.testing.assert_array_equal(p.init[:, -1, 0], x.max(dim=1).values)
    assert torch.all(p.w >= 0.1) and torch.all(p.w <= 1.0)


def test_emeans_uniforms_deterministic_and_in_range():
    a = workloads.emeans_uniforms(7, 16, 1000)
    b = workloads.emeans_uniforms(7, 16, 1000)
    assert a.dtype == np.float32 and a.shape == (16, 1000)
    np.testing.assert_array_equal(a, b)
    assert a.min() >= 0.0 and a.max() < 1.0
    assert not np.array_equal(a, workloads.emeans_uniforms(8, 16, 1000))
    # roughly uniform: mean and quartiles
    assert abs(a.mean() - 0.5) < 0.01
    np.testing.assert_allclose(np.quantile(a, [0.25, 0.5, 0.75]), [0.25, 0.5, 0.75], atol=0.01)


def test_emeans_workload_fields():
    wl = workloads.WORKLOADS["emeans-n1m-k16384-d96-bf16"]
    assert wl.em_batch > 0 and wl.em_epochs > 0 and 0 < wl.em_alpha0 <= 1 and 0 <= wl.em_floor <= 1
    assert wl.N % wl.em_batch == 0 and wl.d == 96 and wl.K == 16384
