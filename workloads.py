"""Seeded synthetic inputs for exact Lloyd k-means, shared by the GPU path and the oracle.

This module only draws random numbers and lays them out; it holds none of the
k-means arithmetic (no distances, no argmin, no means).  Every array is
reproducible from its seed on any machine: numpy's PCG64 generator, with
``SeedSequence.spawn`` children per batch and per fixed-size chunk so the
result does not depend on how many threads generate it.

The shapes and value distributions stand in for the workloads the pages
measure (the pages publish no dataset for them):

* Flash-KMeans articles (technologypulse.uk "Flash-KMeans" article, bottleneck-1
  and performance sections; wispaper.ai "Flash-KMeans" blog, performance
  section): FP16 points, d=128, batched B=32 x N=65536 x K=1024, N=1M x K=8192,
  N=33M x K=4096.
* LeanQuant issue "1D k-means" (github LeanModels/LeanQuant #1, the
  ``kmeans_fit`` diff): per-row weighted 1D clustering of LLM weight rows with
  ``sample_weight`` and a uniform grid init ``linspace(min, max, K)``.

Points are drawn in float32, then rounded to the stored dtype with IEEE
round-to-nearest-even (numpy for fp16, torch CPU for bf16).  Initial
centroids are float32 ``[B, K, d]``.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np
import torch

# Rows generated per independent child seed.  Fixed, so the output does not
# depend on the number of generating threads.
CHUNK_ROWS = 1 << 18

_TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic k-means problem: shapes, distribution and init recipe."""

    name: str
    B: int
    N: int
    d: int
    K: int
    dtype: str              # "f32" | "f16" | "bf16": storage type of the points
    n_iter: int
    seed: int
    kind: str = "gmm"       # "gmm" (Gaussian mixture) | "rows1d" (Student-t rows + weights)
    sigma: float = 0.1      # per-coordinate std of each mixture component
    ncomp: int = 0          # number of mixture components (0: same as K)
    noise_frac: float = 0.0  # fraction of rows replaced by uniform noise
    noise_range: float = 3.0  # noise rows are uniform on [-r, r]^d
    zipf: float = 0.0       # >0: component sizes ~ k^-zipf, k = 1..ncomp
    init: str = "first"     # "first" | "random" | "means_noise" | "linspace"
    init_sigma: float = 0.05  # std of the noise added to the means ("means_noise")
    t_df: float = 4.0       # rows1d: Student-t degrees of freedom
    t_scale: float = 0.02   # rows1d: scale of the t draws
    w_lo: float = 0.1       # rows1d: sample weights ~ U(w_lo, w_hi)
    w_hi: float = 1.0
    host: bool = False      # the points stay in (pinned) host memory: generate_host()
    device_gen: bool = False  # too large for the host generator: generate_device()
    em_batch: int = 0       # e-means: points per step (0: not an e-means workload)
    em_epochs: int = 0      # e-means: passes over the points
    em_alpha0: float = 0.5  # e-means: first step size
    em_floor: float = 0.1   # e-means: last step size as a fraction of the first
    em_dead_frac: float = 0.1  # e-means: dead below this fraction of a batch's mean count per cluster
    em_eps: float = 1e-3    # e-means: relative perturbation of a split

    @property
    def components(self) -> int:
        return self.ncomp if self.ncomp > 0 else self.K

    @property
    def weighted(self) -> bool:
        return self.kind == "rows1d"

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The workloads the library is measured and checked on.  Names state what they are.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("gmm-n8192-k256-d128-f32", B=1, N=8192, d=128, K=256, dtype="f32",
                 n_iter=10, seed=1, sigma=0.1, init="first"),
        Workload("gmm-b32-n65536-k1024-d128-f16", B=32, N=65536, d=128, K=1024, dtype="f16",
                 n_iter=20, seed=2, sigma=0.2, init="random"),
        Workload("gmm-n1m-k8192-d128-f16", B=1, N=1 << 20, d=128, K=8192, dtype="f16",
                 n_iter=10, seed=3, sigma=0.15, noise_frac=0.05, noise_range=3.0,
                 init="random"),
        Workload("zipf-n32m-k4096-d128-bf16", B=1, N=1 << 25, d=128, K=4096, dtype="bf16",
                 n_iter=5, seed=4, sigma=0.15, zipf=1.2, init="means_noise",
                 init_sigma=0.05),
        Workload("rows1d-b4096-n4096-k16-f32", B=4096, N=4096, d=1, K=16, dtype="f32",
                 n_iter=30, seed=5, kind="rows1d", init="linspace"),
        Workload("rows1d-b4096-n4096-k8-f32", B=4096, N=4096, d=1, K=8, dtype="f32",
                 n_iter=30, seed=5, kind="rows1d", init="linspace"),
        Workload("stream-n64m-k32768-d128-f16", B=1, N=1 << 26, d=128, K=32768, dtype="f16",
                 n_iter=3, seed=6, sigma=0.15, init="random", host=True),
        # the out-of-core size of the technologypulse.uk article's performance
        # section, 4e8 points against 16384 centroids (d = 128, 102 GB in
        # fp16): resident in device memory, and streamed from pinned host
        # memory at 2.5e8 points (64 GB, the most one pinned allocation holds
        # on the measuring host)
        Workload("gmm-n400m-k16384-d128-f16", B=1, N=400_000_000, d=128, K=16384, dtype="f16",
                 n_iter=3, seed=8, sigma=0.15, init="random", device_gen=True),
        Workload("stream-n250m-k16384-d128-f16", B=1, N=250_000_000, d=128, K=16384, dtype="f16",
                 n_iter=3, seed=8, sigma=0.15, init="random", host=True),
        # e-means against Lloyd: n_iter is the Lloyd comparison run
        Workload("emeans-n1m-k16384-d96-bf16", B=1, N=1 << 20, d=96, K=16384, dtype="bf16",
                 n_iter=25, seed=7, sigma=0.15, noise_frac=0.05, noise_range=3.0, init="random",
                 em_batch=65536, em_epochs=5, em_alpha0=0.5, em_floor=0.1, em_dead_frac=0.1, em_eps=1e-3),
    ]
}

HEADLINE = "gmm-n1m-k8192-d128-f16"


@dataclasses.dataclass
class Problem:
    """Generated inputs: points, optional weights, initial centroids (CPU tensors)."""

    wl: Workload
    x: torch.Tensor            # [B, N, d], dtype of wl.dtype
    w: torch.Tensor | None     # [B, N] float32 or None
    init: torch.Tensor         # [B, K, d] float32
    means: np.ndarray | None = None  # [B, ncomp, d] float64 component means (gmm only)


def _to_dtype(a32: np.ndarray, dtype: str) -> torch.Tensor:
    """Round a float32 array to the storage dtype (IEEE round-to-nearest-even)."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    if dtype == "f16":
        return torch.from_numpy(a32.astype(np.float16))
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16)
    raise ValueError(dtype)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _gmm_batch(wl: Workload, ss: np.random.SeedSequence, out: torch.Tensor):
    """Fill out[N, d] with one batch of the Gaussian mixture; return the means."""
    ss_means, ss_comp, ss_pts, ss_noise = ss.spawn(4)
    N, d, m = wl.N, wl.d, wl.components
    means = np.random.default_rng(ss_means).standard_normal((m, d))  # float64
    rng_c = np.random.default_rng(ss_comp)
    if wl.zipf > 0:
        p = np.arange(1, m + 1, dtype=np.float64) ** (-wl.zipf)
        p /= p.sum()
        comp = rng_c.choice(m, size=N, p=p).astype(np.int32)
    else:
        comp = rng_c.integers(0, m, size=N, dtype=np.int32)
    n_noise = int(round(wl.noise_frac * N))
    noise_rows = None
    if n_noise > 0:
        rng_n = np.random.default_rng(ss_noise)
        noise_rows = np.sort(rng_n.choice(N, size=n_noise, replace=False))
        noise_vals = rng_n.uniform(-wl.noise_range, wl.noise_range, size=(n_noise, d)).astype(np.float32)
    means32 = means.astype(np.float32)
    nchunks = (N + CHUNK_ROWS - 1) // CHUNK_ROWS
    chunk_ss = ss_pts.spawn(nchunks)
    sigma = np.float32(wl.sigma)

    def work(c):
        lo, hi = c * CHUNK_ROWS, min(N, (c + 1) * CHUNK_ROWS)
        z = np.random.default_rng(chunk_ss[c]).standard_normal((hi - lo, d), dtype=np.float32)
        z *= sigma
        z += means32[comp[lo:hi]]
        if noise_rows is not None:
            a, b = np.searchsorted(noise_rows, [lo, hi])
            if b > a:
                z[noise_rows[a:b] - lo] = noise_vals[a:b]
        out[lo:hi].copy_(_to_dtype(z, wl.dtype))

    if nchunks == 1:
        work(0)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return means


def _rows1d_batch(wl: Workload, ss: np.random.SeedSequence):
    ss_x, ss_w = ss.spawn(2)
    x = (wl.t_scale * np.random.default_rng(ss_x).standard_t(wl.t_df, size=wl.N)).astype(np.float32)
    w = np.random.default_rng(ss_w).uniform(wl.w_lo, wl.w_hi, size=wl.N).astype(np.float32)
    return x, w


def generate(wl: Workload) -> Problem:
    """Generate the points, weights and initial centroids of a workload."""
    root = np.random.SeedSequence(wl.seed)
    ss_data, ss_init = root.spawn(2)
    batch_ss = ss_data.spawn(wl.B)
    init_ss = ss_init.spawn(wl.B)
    x = torch.empty((wl.B, wl.N, wl.d), dtype=_TORCH_DTYPE[wl.dtype])
    w = None
    means = None
    if wl.kind == "gmm":
        means = np.empty((wl.B, wl.components, wl.d), dtype=np.float64)
        for b in range(wl.B):
            means[b] = _gmm_batch(wl, batch_ss[b], x[b])
    elif wl.kind == "rows1d":
        if wl.d != 1:
            raise ValueError("rows1d workloads have d == 1")
        w = torch.empty((wl.B, wl.N), dtype=torch.float32)

        def work(b):
            xb, wb = _rows1d_batch(wl, batch_ss[b])
            x[b, :, 0].copy_(torch.from_numpy(xb))
            w[b].copy_(torch.from_numpy(wb))

        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(wl.B)))
    else:
        raise ValueError(wl.kind)
    init = make_init(wl, x, means, init_ss)
    return Problem(wl, x, w, init, means)


def make_init(wl: Workload, x: torch.Tensor, means, init_ss) -> torch.Tensor:
    """Initial centroids [B, K, d] float32 by the workload's init recipe.

    * ``first``: rows 0..K-1 of each batch.
    * ``random``: K distinct rows per batch, drawn without replacement.
    * ``means_noise``: the mixture means plus N(0, init_sigma^2) noise.
    * ``linspace``: K values evenly spaced from the row minimum to the row
      maximum, endpoints included (the uniform grid init of the LeanQuant
      "1D k-means" issue); d must be 1.
    """
    B, N, d, K = wl.B, wl.N, wl.d, wl.K
    init = torch.empty((B, K, d), dtype=torch.float32)
    if wl.init == "first":
        if K > N:
            raise ValueError("first-K init needs K <= N")
        init.copy_(x[:, :K, :].float())
    elif wl.init == "random":
        if K > N:
            raise ValueError("random-K init needs K <= N")
        for b in range(B):
            idx = np.random.default_rng(init_ss[b]).choice(N, size=K, replace=False)
            init[b].copy_(x[b, torch.from_numpy(idx)].float())
    elif wl.init == "means_noise":
        if means is None or means.shape[1] != K:
            raise ValueError("means_noise init needs ncomp == K")
        for b in range(B):
            e = np.random.default_rng(init_ss[b]).standard_normal((K, d))
            init[b].copy_(torch.from_numpy((means[b] + wl.init_sigma * e).astype(np.float32)))
    elif wl.init == "linspace":
        if d != 1:
            raise ValueError("linspace init is for d == 1")
        xf = x[:, :, 0].double().numpy()
        lo, hi = xf.min(axis=1), xf.max(axis=1)
        grid = np.linspace(lo, hi, num=K, axis=1)  # [B, K]
        init[:, :, 0].copy_(torch.from_numpy(grid.astype(np.float32)))
    else:
        raise ValueError(wl.init)
    return init


def small(name: str, **kw) -> Workload:
    """A reduced copy of a named workload (for tests that run the oracle in full)."""
    return WORKLOADS[name].replace(**kw)


def raw_bits(x: torch.Tensor) -> np.ndarray:
    """Stored bits of a CPU tensor as numpy: float32 stays float32, fp16/bf16 become uint16."""
    if x.dtype == torch.float32:
        return x.contiguous().numpy()
    if x.dtype in (torch.float16, torch.bfloat16):
        return x.contiguous().view(torch.int16).numpy().view(np.uint16)
    raise TypeError(x.dtype)


def dtype_name(x: torch.Tensor) -> str:
    return {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[x.dtype]


def _gmm_on_gpu(wl: Workload, x: torch.Tensor, chunk: int) -> torch.Tensor:
    """Fill x [N, d] (host or device) with a Gaussian mixture made on the GPU
    from a seeded generator (numpy would take minutes at these sizes):
    wl.components means ~ N(0, 1), per-coordinate std wl.sigma, components
    drawn uniformly, stored in wl.dtype.  Returns the indices of K distinct
    random points (the initial centroids)."""
    g = torch.Generator(device="cuda").manual_seed(wl.seed)
    means = torch.randn((wl.components, wl.d), generator=g, device="cuda")
    for p0 in range(0, wl.N, chunk):
        n = min(chunk, wl.N - p0)
        comp = torch.randint(0, wl.components, (n,), generator=g, device="cuda")
        v = means[comp] + wl.sigma * torch.randn((n, wl.d), generator=g, device="cuda")
        x[p0:p0 + n].copy_(v.to(_TORCH_DTYPE[wl.dtype]))
    return torch.randperm(wl.N, generator=g, device="cuda")[:wl.K]


def generate_host(wl: Workload, chunk: int = 1 << 22):
    """Points of a host-memory workload (_gmm_on_gpu, copied into pinned host
    memory).  Returns (x_host [N, d] pinned CPU tensor, init [K, d] float32
    on the GPU: K distinct random points)."""
    assert wl.host and wl.B == 1 and wl.kind == "gmm"
    x = torch.empty((wl.N, wl.d), dtype=_TORCH_DTYPE[wl.dtype], pin_memory=True)
    idx = _gmm_on_gpu(wl, x, chunk).cpu()
    init = x[idx].float().cuda()
    torch.cuda.synchronize()
    return x, init


def generate_device(wl: Workload, chunk: int = 1 << 22):
    """Points of a workload made and kept on the GPU (_gmm_on_gpu).  Returns
    (x [1, N, d] in device memory, init [1, K, d] float32: K distinct random
    points)."""
    assert wl.device_gen and wl.B == 1 and wl.kind == "gmm"
    x = torch.empty((1, wl.N, wl.d), dtype=_TORCH_DTYPE[wl.dtype], device="cuda")
    idx = _gmm_on_gpu(wl, x[0], chunk)
    init = x[0, idx].float()[None].contiguous()
    torch.cuda.synchronize()
    return x, init


def emeans_uniforms(seed: int, steps: int, K: int) -> np.ndarray:
    """The split draws of an e-means run: [steps, K] float32 uniform on
    [0, 1), from their own seed sequence (entropy [seed, 7919])."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 7919]))
    return rng.random((steps, K), dtype=np.float32)
