"""Seeded synthetic workloads for the FVAttn block-sparse attention hot path.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic (no pooling, scoring, selection or attention), so both the
CPU oracle and the HIP path can take their inputs from it without sharing any
of the computation under test.

Workload shapes follow the FVAttn pages (arXiv 2607.16190): a 720p Wan2.2-14B
image-to-video latent is a 21x45x80 token grid with 40 heads of width 128
(paperlayer.ai summary, section 1 "Introduction", the H20 motivation remark);
one rank of eight owns 5 of those heads (section 3, "Runtime Load Balancing",
the 8-GPU migration-budget remark).  The pages measure on trained Wan2.2
activations, which are not available here; the random-Fourier-feature
generator below stands in for them (see ``make_inputs``).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

SEED = 260716190          # arXiv id 2607.16190 without the dot
RFF_BANDWIDTH = 0.3       # sigma of the random Fourier features
NOISE_STD = 0.5           # i.i.d. noise added to q and k


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic attention layer.

    grid  = (T, Y, X) latent tokens; token index n = (t*Y + y)*X + x.
    tile  = (tt, ty, tx) 3D tile that forms one block.
    budget = ("none", 0.0) | ("frac", f) | ("match_max", 0.0).
    gains = fixed per-head gains, or None for log-uniform draws in [0.5, 4].
    """
    cid: int
    name: str
    B: int
    H: int
    d: int
    dtype: str            # "fp32" | "bf16"
    grid: Tuple[int, int, int]
    tile: Tuple[int, int, int]
    p: float
    kmin: int
    budget: Tuple[str, float]
    gains: Optional[Tuple[float, ...]]
    temporal: float       # weight of the temporal-locality term
    sample_qblocks: int = 0   # >0: oracle attention checks this many query blocks per head

    @property
    def N(self) -> int:
        T, Y, X = self.grid
        return T * Y * X

    def with_heads(self, H: int, gains: Optional[Sequence[float]] = None) -> "Workload":
        return dataclasses.replace(self, H=H, gains=tuple(gains) if gains is not None else self.gains)


WORKLOADS = {
    1: Workload(1, "tiny-fp32", 1, 2, 64, "fp32", (4, 8, 8), (1, 8, 8), 0.9, 1,
                ("none", 0.0), (0.5, 3.0), 0.0),
    2: Workload(2, "mid-bf16", 1, 12, 128, "bf16", (5, 30, 52), (2, 8, 8), 0.9, 4,
                ("frac", 0.10), None, 0.0),
    3: Workload(3, "720p-layer", 1, 40, 128, "bf16", (21, 45, 80), (2, 8, 8), 0.9, 8,
                ("frac", 0.10), None, 0.3),
    4: Workload(4, "720p-5head-shard", 1, 5, 128, "bf16", (21, 45, 80), (2, 8, 8), 0.9, 8,
                ("match_max", 0.0), (0.3, 0.3, 0.5, 3.0, 4.0), 0.3),
    5: Workload(5, "1080p-layer", 1, 40, 128, "bf16", (21, 68, 120), (2, 8, 8), 0.95, 16,
                ("frac", 0.05), None, 0.0, sample_qblocks=64),
}


def head_gains(w: Workload, rng: np.random.Generator) -> np.ndarray:
    """Per-(batch, head) gains a_h: fixed list, or exp(U[ln 0.5, ln 4])."""
    if w.gains is not None:
        g = np.asarray(w.gains, dtype=np.float64)
        assert g.shape == (w.H,)
        return np.tile(g, (w.B, 1))
    return np.exp(rng.uniform(math.log(0.5), math.log(4.0), size=(w.B, w.H)))


def _grid_coords(grid):
    T, Y, X = grid
    t, y, x = np.meshgrid(np.arange(T), np.arange(Y), np.arange(X), indexing="ij")
    u = np.stack([t.ravel() / T, y.ravel() / Y, x.ravel() / X], axis=1)   # [N, 3]
    return u, t.ravel() / T


def make_inputs(w: Workload, heads: Optional[Sequence[int]] = None, seed: int = SEED):
    """Return (q, k, v, gains) as CPU torch tensors [B, H', N, d] in the workload dtype.

    Recipe (seeded with default_rng((seed, cid)); draws in this order):
      1. gains a_{b,h}: the fixed list, or log-uniform in [0.5, 4];
      2. Omega [d, 3] ~ N(0, 1/sigma^2), beta [d] ~ U[0, 2pi), sigma = 0.3;
      3. if temporal > 0: omega' [d] ~ N(0, 1/sigma^2), beta' [d] ~ U[0, 2pi);
      4. per (b, h) in order: eps_q, eps_k, v, each [N, d] ~ N(0, 1) in float32.
    phi(u) = sqrt(2) cos(Omega u + beta) with u = (t/T, y/Y, x/X) (unit-variance
    features); psi(t) = sqrt(2) cos(omega' t/T + beta').
    q = a phi + w_t psi + 0.5 eps_q, k likewise with eps_k; computed in float32
    and rounded to bf16 (round-to-nearest-even) for bf16 workloads.

    ``heads`` selects a subset of heads (the draws for the others are still made,
    so a subset is bit-identical to the same heads of the full tensor).
    """
    import torch

    rng = np.random.default_rng((seed, w.cid))
    gains = head_gains(w, rng)
    omega = rng.normal(0.0, 1.0 / RFF_BANDWIDTH, size=(w.d, 3))
    beta = rng.uniform(0.0, 2.0 * math.pi, size=w.d)
    if w.temporal > 0:
        omega_t = rng.normal(0.0, 1.0 / RFF_BANDWIDTH, size=w.d)
        beta_t = rng.uniform(0.0, 2.0 * math.pi, size=w.d)
    u, tn = _grid_coords(w.grid)
    phi = (math.sqrt(2.0) * np.cos(u @ omega.T + beta)).astype(np.float32)          # [N, d]
    if w.temporal > 0:
        psi = (math.sqrt(2.0) * np.cos(np.outer(tn, omega_t) + beta_t)).astype(np.float32)
        base_t = np.float32(w.temporal) * psi
    else:
        base_t = None

    hsel = list(range(w.H)) if heads is None else list(heads)
    tdtype = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    q = torch.empty((w.B, len(hsel), w.N, w.d), dtype=tdtype)
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    pos = {h: i for i, h in enumerate(hsel)}
    for b in range(w.B):
        for h in range(w.H):
            eq = rng.standard_normal((w.N, w.d), dtype=np.float32)
            ek = rng.standard_normal((w.N, w.d), dtype=np.float32)
            ev = rng.standard_normal((w.N, w.d), dtype=np.float32)
            if h not in pos:
                continue
            a = np.float32(gains[b, h])
            qh = a * phi + np.float32(NOISE_STD) * eq
            kh = a * phi + np.float32(NOISE_STD) * ek
            if base_t is not None:
                qh += base_t
                kh += base_t
            j = pos[h]
            q[b, j] = torch.from_numpy(qh).to(tdtype)
            k[b, j] = torch.from_numpy(kh).to(tdtype)
            v[b, j] = torch.from_numpy(ev).to(tdtype)
    return q, k, v, gains[:, hsel]


def sample_qblocks(w: Workload, nq: int, seed: int = SEED) -> List[np.ndarray]:
    """Seeded per-head sample of query blocks for sampled parity checks."""
    rng = np.random.default_rng((seed, w.cid, 1))
    n = min(w.sample_qblocks or nq, nq)
    return [np.sort(rng.choice(nq, n, replace=False)) for _ in range(w.B * w.H)]


def tiny_random(shape, seed, dtype="fp32", scale=1.0):
    """Small seeded N(0, scale^2) tensor for unit tests (CPU torch)."""
    import torch
    rng = np.random.default_rng(seed)
    x = (scale * rng.standard_normal(shape)).astype(np.float32)
    t = torch.from_numpy(x)
    return t if dtype == "fp32" else t.to(torch.bfloat16)
