"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the benchmark.

This module models the *workload* only: temporally correlated activations and
low-rank-plus-noise matrices at the shapes of FLUX.1-dev and CogVideoX-2b
exchanges.  It contains none of the codec's or the subspace iteration's
arithmetic, so the CPU oracle and the HIP path can both consume its output
without sharing any method code.

Workload model (the pages only say that adjacent denoising steps produce
highly similar activations -- "Accelerating Parallel Diffusion Model Serving
with Residual Compression", abstract -- so a stationary AR(1) process stands in
for that temporal redundancy):

* per tensor channel scales  sc_c = exp(0.5 * z_c),  z ~ N(0, 1)  (LogNormal(0, 0.5));
  optionally round(frac * cols) channels, picked by a seeded permutation, are
  multiplied by ``outlier_mult``;
* X_0 = N(0, 1) * sc;   X_t = alpha * X_{t-1} + noise * N(0, 1) * sc;
* the state is kept in fp32 and every X_t is emitted as bf16 (round to nearest even).

Low-rank inputs: A = F G^T + sigma * N(0, 1) with Gaussian factors, emitted as bf16,
plus a Gaussian starting block Q0 (the random sample of the subspace iteration,
drawn here so that every implementation sees identical bits).
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass

import torch

__all__ = [
    "WorkloadSpec",
    "SPECS",
    "seed_for",
    "AR1Stream",
    "lowrank_batch",
    "exact_rank_batch",
    "gaussian_q0",
]


def seed_for(*key) -> int:
    """A 63-bit seed derived from an arbitrary key tuple (stable across runs and hosts)."""
    h = hashlib.sha256(repr(key).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


@dataclass(frozen=True)
class WorkloadSpec:
    """One exchanged-activation workload: ``tensors`` independent (layer, K|V) streams."""

    name: str
    tensors: int          # layers x {K, V}
    rows: int             # tokens held by this GPU
    cols: int             # channels
    steps: int            # denoising steps (step 0 is the uncompressed warm-up)
    alpha: float          # AR(1) coefficient
    noise: float          # AR(1) innovation scale
    outlier_frac: float   # fraction of channels given an outlier scale
    outlier_mult: float = 20.0

    @property
    def elems_per_tensor(self) -> int:
        return self.rows * self.cols

    @property
    def elems_per_step(self) -> int:
        return self.tensors * self.rows * self.cols


# The workloads named by the configurations this library is measured on.
SPECS = {
    # 256 tokens x 512 channels, one tensor, 4 steps, no outliers.
    "tiny": WorkloadSpec("tiny", 1, 256, 512, 4, 0.98, 0.199, 0.0),
    # FLUX.1-dev at patch degree 4: K and V of 57 layers, 1024 tokens x 3072 channels, 28 steps.
    "flux": WorkloadSpec("flux", 114, 1024, 3072, 28, 0.98, 0.199, 0.01),
    # CogVideoX-2b sequence-parallel share at degree 4: 30 layers, 4388 tokens x 1920, 50 steps.
    # The innovation scale sqrt(1 - 0.97^2) keeps the process stationary, as 0.199 does for 0.98.
    "cogvideox": WorkloadSpec("cogvideox", 60, 4388, 1920, 50, 0.97, 0.2431, 0.01),
}


class AR1Stream:
    """Seeded AR(1) activations for ``n_tensors`` streams of shape ``rows x cols``.

    ``next()`` returns X_0, X_1, ... as a bf16 tensor ``[n_tensors, rows, cols]`` on
    ``device``.  The draws depend on (seed, key) and on the device's generator
    (torch's CPU and GPU generators give different streams), never on anything else.
    """

    def __init__(self, n_tensors, rows, cols, alpha, noise, outlier_frac=0.0,
                 outlier_mult=20.0, seed=0, key="ar1", device="cpu"):
        self.shape = (n_tensors, rows, cols)
        self.alpha = float(alpha)
        self.noise = float(noise)
        self.device = torch.device(device)
        self.gen = torch.Generator(device=self.device)
        self.gen.manual_seed(seed_for(seed, key, n_tensors, rows, cols))
        z = torch.randn((n_tensors, 1, cols), generator=self.gen, device=self.device)
        sc = torch.exp(0.5 * z)
        n_out = int(round(outlier_frac * cols))
        if n_out > 0:
            for i in range(n_tensors):
                perm = torch.randperm(cols, generator=self.gen, device=self.device)
                sc[i, 0, perm[:n_out]] *= outlier_mult
        self.scales = sc
        self.state = None
        self.t = -1

    @classmethod
    def from_spec(cls, spec: WorkloadSpec, seed=0, device="cpu", n_tensors=None, rows=None):
        return cls(n_tensors or spec.tensors, rows or spec.rows, spec.cols, spec.alpha,
                   spec.noise, spec.outlier_frac, spec.outlier_mult, seed=seed,
                   key=spec.name, device=device)

    def next(self) -> torch.Tensor:
        eps = torch.randn(self.shape, generator=self.gen, device=self.device)
        if self.state is None:
            self.state = eps * self.scales
        else:
            self.state = self.alpha * self.state + self.noise * (eps * self.scales)
        self.t += 1
        return self.state.to(torch.bfloat16)


def gaussian_q0(batch, n, r, seed=0, key="q0", device="cpu") -> torch.Tensor:
    """The random starting block of the subspace iteration, N(0, 1) fp32 ``[batch, n, r]``."""
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(seed, key, batch, n, r))
    return torch.randn((batch, n, r), generator=g, device=device, dtype=torch.float32)


def lowrank_batch(batch, m, n, rank=16, sigma=0.05, seed=0, key="lowrank", device="cpu"):
    """``batch`` matrices A = F G^T + sigma * N(0, 1), F: m x rank, G: n x rank Gaussian, as bf16."""
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(seed, key, batch, m, n, rank))
    f = torch.randn((batch, m, rank), generator=g, device=device)
    gg = torch.randn((batch, n, rank), generator=g, device=device)
    a = torch.bmm(f, gg.transpose(1, 2).contiguous()) if rank > 0 else torch.zeros(
        (batch, m, n), device=device)
    a = a + sigma * torch.randn((batch, m, n), generator=g, device=device)
    return a.to(torch.bfloat16)


def graded_batch(batch, m, n, k=48, decades=4.0, seed=0, key="graded", device="cpu"):
    """Ill-conditioned inputs: A = F diag(s) G^T with F (m x k), G (n x k) Gaussian and
    s_i = 10^(-decades * i / (k - 1)), i < k -- a spectrum that falls geometrically over
    ``decades`` decades -- as bf16 (built in fp64 on the CPU, then moved to ``device``)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed_for(seed, key, batch, m, n, k, int(decades * 1000)))
    f = torch.randn((batch, m, k), generator=g, dtype=torch.float64)
    gg = torch.randn((batch, n, k), generator=g, dtype=torch.float64)
    s = torch.pow(10.0, -decades * torch.arange(k, dtype=torch.float64) / max(k - 1, 1))
    a = torch.bmm(f * s, gg.transpose(1, 2).contiguous())
    return a.to(torch.bfloat16).to(device)


def exact_rank_batch(batch, m, n, rank, seed=0, key="exact", device="cpu"):
    """A = F G^T with F, G entries in {-1, 0, 1}: every entry is an integer of size <= rank,
    so A is exactly representable in bf16 for rank <= 256 and has rank <= ``rank`` exactly."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed_for(seed, key, batch, m, n, rank))
    f = torch.randint(-1, 2, (batch, m, rank), generator=g).to(torch.float64)
    gg = torch.randint(-1, 2, (batch, n, rank), generator=g).to(torch.float64)
    a = torch.bmm(f, gg.transpose(1, 2).contiguous())
    return a.to(torch.bfloat16).to(device)


class LowrankDrift:
    """Activations whose step-to-step change is low-rank plus noise, ``[batch, rows, cols]`` bf16.

    X_0 = N(0, 1); X_t = X_{t-1} + c * (F_t G_t^T / sqrt(rank) + sigma * N(0, 1)) with F_t
    (rows x rank) and G_t (cols x rank) Gaussian, drawn afresh every step.  The generator keeps
    X in fp32 and emits it rounded to bf16.  The first call of ``next`` returns X_0."""

    def __init__(self, batch, rows, cols, rank=16, sigma=0.05, c=0.2, seed=0, key="lrdrift",
                 device="cpu"):
        self.batch, self.rows, self.cols = batch, rows, cols
        self.rank, self.sigma, self.c = rank, sigma, c
        self.device = device
        self.g = torch.Generator(device=device)
        self.g.manual_seed(seed_for(seed, key, batch, rows, cols, rank))
        self.x = None

    def next(self) -> torch.Tensor:
        shape = (self.batch, self.rows, self.cols)
        if self.x is None:
            self.x = torch.randn(shape, generator=self.g, device=self.device)
        else:
            f = torch.randn((self.batch, self.rows, self.rank), generator=self.g, device=self.device)
            gg = torch.randn((self.batch, self.cols, self.rank), generator=self.g,
                             device=self.device)
            inc = torch.bmm(f, gg.transpose(1, 2).contiguous()) / math.sqrt(self.rank)
            inc += self.sigma * torch.randn(shape, generator=self.g, device=self.device)
            self.x += self.c * inc
        return self.x.to(torch.bfloat16)
