"""Seeded synthetic inputs for the routed sparse-attention path.

This module only draws random numbers and shapes them into activations with
the structure of the workloads the SVG-EAR pages evaluate on (video DiT
attention over a latent grid, pages: arXiv 2603.08982 HTML, section 5
"Models"). It holds none of the method's arithmetic and is shared by the
CPU oracle tests and the HIP path, so both see identical inputs.

Every tensor is generated per head from ``numpy.random.default_rng`` seeded
with a ``SeedSequence`` that names the head and the tensor, so a single head
can be regenerated without the others (used to time and check one head of a
40-head layer). bf16 inputs are rounded once, round-to-nearest-even, by
torch on the CPU; both sides then read the same values.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

TENSOR_Q, TENSOR_K, TENSOR_V = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and generator parameters of one attention layer."""

    name: str
    heads: int
    n: int                 # N_q = N_k
    d: int
    dtype: str             # "f32" or "bf16"
    cq: int
    ck: int
    rho: float
    iters: int
    gen: str               # "blobs" | "lattice" | "stress"
    centres: int
    sigma: float
    zipf: float = 0.0      # 0 -> uniform latent choice
    grid: tuple = ()       # (frames, rows, cols) for the lattice generator
    outlier_frac: float = 0.0
    outlier_sigma: float = 0.0
    seed: int = 0

    @property
    def budget(self) -> int:
        """Exact keys each query cluster may attend to: floor(rho * N_k)."""
        return int(math.floor(self.rho * self.n))

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1024, 64, "f32", 16, 16, 0.25, 10, "blobs", 16, 0.3),
    "slice": Workload("slice", 8, 16384, 128, "bf16", 100, 500, 0.15, 10, "blobs", 256,
                      0.25, zipf=1.1),
    "wan22": Workload("wan22", 40, 21 * 45 * 80, 128, "bf16", 100, 500, 0.10, 10, "lattice",
                      512, 0.25, grid=(21, 45, 80)),
    "hunyuan": Workload("hunyuan", 24, 33 * 45 * 80, 128, "bf16", 100, 500, 0.10, 10,
                        "lattice", 512, 0.25, grid=(33, 45, 80)),
    "stress": Workload("stress", 40, 21 * 45 * 80, 128, "bf16", 100, 500, 0.10, 10, "stress",
                       1000, 0.25, zipf=1.5, outlier_frac=0.05, outlier_sigma=1.0),
}


def _rng(*ids: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(list(ids)))


def _zipf_probs(k: int, s: float) -> np.ndarray:
    p = np.arange(1, k + 1, dtype=np.float64) ** (-s)
    return p / p.sum()


_LATTICE_CACHE: dict = {}


def _lattice_weights(grid: tuple) -> np.ndarray:
    """[N, 512] float32 smoothing weights of each grid token to an 8x8x8 lattice.

    A token at (t, h, w) sits at u = ((t+1/2)/T, (h+1/2)/Hh, (w+1/2)/W) in the
    unit cube; lattice point (i, j, k) sits at ((i+1/2)/8, ...). The weight is a
    Gaussian of the distance with bandwidth one lattice spacing, normalised so
    that a sum of unit-variance centres keeps unit variance per dimension.
    """
    if grid in _LATTICE_CACHE:
        return _LATTICE_CACHE[grid]
    T, Hh, W = grid
    t, h, w = np.meshgrid((np.arange(T) + 0.5) / T, (np.arange(Hh) + 0.5) / Hh,
                          (np.arange(W) + 0.5) / W, indexing="ij")
    u = np.stack([t.ravel(), h.ravel(), w.ravel()], axis=1)              # [N, 3]
    a = (np.arange(8) + 0.5) / 8
    li, lj, lk = np.meshgrid(a, a, a, indexing="ij")
    lat = np.stack([li.ravel(), lj.ravel(), lk.ravel()], axis=1)         # [512, 3]
    s = 1.0 / 8
    d2 = ((u[:, None, :] - lat[None, :, :]) ** 2).sum(-1)
    wts = np.exp(-d2 / (2 * s * s))
    wts /= np.sqrt((wts ** 2).sum(1, keepdims=True))
    out = wts.astype(np.float32)
    _LATTICE_CACHE[grid] = out
    return out


def _latent(wl: Workload, head: int):
    """Per-token latent draws shared by the Q, K and V rows of one head."""
    rng = _rng(wl.seed, head, 99)
    n = wl.n
    z = None
    if wl.gen in ("blobs", "stress"):
        if wl.zipf > 0:
            z = rng.choice(wl.centres, size=n, p=_zipf_probs(wl.centres, wl.zipf))
        else:
            z = rng.integers(0, wl.centres, size=n)
    outlier = np.zeros(n, dtype=bool)
    if wl.outlier_frac > 0:
        idx = rng.choice(n, size=int(round(wl.outlier_frac * n)), replace=False)
        outlier[idx] = True
    return z, outlier


def head_tensor(wl: Workload, head: int, tensor_id: int, z=None, outlier=None) -> np.ndarray:
    """One head of Q (0), K (1) or V (2) as float32 [N, d], before rounding."""
    if z is None and outlier is None:
        z, outlier = _latent(wl, head)
    rng = _rng(wl.seed, head, tensor_id)
    d = wl.d
    if wl.gen == "lattice":
        centres = rng.standard_normal((wl.centres, d), dtype=np.float32)
        mean = _lattice_weights(wl.grid) @ centres
    else:
        centres = rng.standard_normal((wl.centres, d), dtype=np.float32)
        mean = centres[z]
    noise = rng.standard_normal((wl.n, d), dtype=np.float32)
    sig = np.full((wl.n, 1), wl.sigma, dtype=np.float32)
    if outlier is not None and outlier.any():
        sig[outlier] = wl.outlier_sigma
    return (mean + sig * noise).astype(np.float32)


def _round(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(x)
    return t.to(torch.bfloat16) if dtype == "bf16" else t.clone()


def make_qkv(wl: Workload, heads=None, threads: int = 8):
    """Q, K, V as CPU torch tensors [H', N, d] in the workload dtype.

    ``heads`` selects a subset of head indices (default: all); each head is
    generated independently, so a subset equals the same rows of the full set.
    """
    heads = list(range(wl.heads)) if heads is None else list(heads)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    out = [torch.empty((len(heads), wl.n, wl.d), dtype=tdt) for _ in range(3)]

    def one(i_h):
        i, h = i_h
        z, outl = _latent(wl, h)
        for tid in range(3):
            out[tid][i] = _round(head_tensor(wl, h, tid, z, outl), wl.dtype)

    if wl.gen == "lattice":
        _lattice_weights(wl.grid)
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(one, enumerate(heads)))
    return out[0], out[1], out[2]


def kmeans_init(x: torch.Tensor, c: int, seed: int, tensor_id: int, head_ids=None) -> torch.Tensor:
    """Initial centroids: C distinct rows of each head, drawn without replacement.

    ``x`` is [H', N, d] (any dtype); returns float32 [H', C, d] holding the
    chosen rows exactly. ``head_ids`` names the original head index of each
    slice so a subset of heads draws the same rows as the full tensor.
    """
    hs = x.shape[0]
    head_ids = list(range(hs)) if head_ids is None else list(head_ids)
    out = torch.empty((hs, c, x.shape[2]), dtype=torch.float32)
    for i, h in enumerate(head_ids):
        idx = _rng(seed, 10 + tensor_id, h).choice(x.shape[1], size=c, replace=False)
        out[i] = x[i, torch.from_numpy(np.sort(idx))].float()
    return out
