"""Seeded synthetic inputs for the Dion3 optimizer step.

This module only draws random matrices; it holds none of the method's
arithmetic (no scoring, selection, orthogonalization or update).  Both the
fp64 oracle (through the tests) and the HIP path consume what it produces,
so the two sides always see the same fp32 bytes.

Workloads (the shapes are those of dense transformer weight sets; the pages
train on ClimbMix, whose trained momenta are not available, so seeded
Gaussian or low-rank matrices of the same shapes stand in for them):

* ``c1``  one 128x512 momentum matrix, f = 1/4.
* ``c2``  16 matrices of 1024x4096, f = 1 (the full-matrix, Muon-equivalent path).
* ``c3``  1B-like set: hidden 2048, 24 layers (Q/K/V/O 2048x2048, gate/up
          5504x2048, down 2048x5504); per-matrix scale U(0.1, 10); f = 1/4.
* ``c4``  7B-like set: hidden 4096, 32 layers (4 x 4096x4096,
          2 x 11008x4096, 1 x 4096x11008); f = 1/2 or 1/4.
* ``c5``  14B-like set: hidden 5120, 40 layers (4 x 5120x5120,
          2 x 13824x5120, 1 x 5120x13824); ill-conditioned momentum
          (rank-64 part with singular values i^-1.5 plus relative 1e-3
          Frobenius noise); f = 1/8.

Small inputs are drawn on the host with NumPy's PCG64; the large weight sets
are drawn on the device with ``torch.Generator`` so that the 7B and 14B sets
(52 GB and 102 GB of fp32 state) never pass through host memory.
"""
from __future__ import annotations

import dataclasses
import math
from fractions import Fraction
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

# The Muon-style learning-rate base; the step uses eta = LR_BASE / sqrt(f).
LR_BASE = 0.02
MU = 0.95
W_STD = 0.02


@dataclasses.dataclass(frozen=True)
class ShapeGroup:
    """``count`` matrices of shape ``n x m`` (rows = output neurons)."""
    count: int
    n: int
    m: int


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    groups: Tuple[ShapeGroup, ...]
    fraction: Fraction
    kind: str            # "gaussian", "scaled" or "lowrank"
    seed_base: int

    @property
    def lr(self) -> float:
        return LR_BASE / math.sqrt(float(self.fraction))

    @property
    def n_matrices(self) -> int:
        return sum(g.count for g in self.groups)

    @property
    def n_params(self) -> int:
        return sum(g.count * g.n * g.m for g in self.groups)


def _model_groups(hidden: int, mlp: int, layers: int) -> Tuple[ShapeGroup, ...]:
    return (ShapeGroup(4 * layers, hidden, hidden),
            ShapeGroup(2 * layers, mlp, hidden),
            ShapeGroup(1 * layers, hidden, mlp))


WORKLOADS: Dict[str, Workload] = {
    "c1": Workload("c1-128x512-f1/4", (ShapeGroup(1, 128, 512),), Fraction(1, 4), "gaussian", 0),
    "c2": Workload("c2-16x1024x4096-f1", (ShapeGroup(16, 1024, 4096),), Fraction(1, 1), "gaussian", 0),
    "c3": Workload("c3-1B-f1/4", _model_groups(2048, 5504, 24), Fraction(1, 4), "scaled", 3000),
    "c4h": Workload("c4-7B-f1/2", _model_groups(4096, 11008, 32), Fraction(1, 2), "gaussian", 4000),
    "c4": Workload("c4-7B-f1/4", _model_groups(4096, 11008, 32), Fraction(1, 4), "gaussian", 4000),
    "c4f": Workload("c4-7B-f1", _model_groups(4096, 11008, 32), Fraction(1, 1), "gaussian", 4000),
    "c5": Workload("c5-14B-f1/8", _model_groups(5120, 13824, 40), Fraction(1, 8), "lowrank", 5000),
}


# ---------------------------------------------------------------- host side

def host_gaussian(shape: Sequence[int], seed, std: float = 1.0) -> np.ndarray:
    """fp32 N(0, std^2) matrix from PCG64 seeded with ``seed`` (int or list)."""
    rng = np.random.default_rng(seed)
    if std == 1.0:
        return rng.standard_normal(tuple(shape)).astype(np.float32)
    return rng.normal(0.0, std, tuple(shape)).astype(np.float32)


def c1_inputs() -> Tuple[np.ndarray, np.ndarray]:
    """The single 128x512 case: M ~ N(0,1) seed 0, W ~ N(0, 0.02^2) seed 1."""
    m = np.random.default_rng(0).standard_normal((128, 512)).astype(np.float32)
    w = np.random.default_rng(1).normal(0.0, W_STD, (128, 512)).astype(np.float32)
    return w, m


def c2_inputs(batch: int = 16, n: int = 1024, m: int = 4096) -> Tuple[np.ndarray, np.ndarray]:
    """Batch of same-shape matrices: M_b ~ N(0,1) seed [0,b], W_b ~ N(0,0.02^2) seed [1,b]."""
    ms = np.stack([np.random.default_rng([0, b]).standard_normal((n, m)).astype(np.float32)
                   for b in range(batch)])
    ws = np.stack([np.random.default_rng([1, b]).normal(0.0, W_STD, (n, m)).astype(np.float32)
                   for b in range(batch)])
    return ws, ms


def host_lowrank(n: int, m: int, seed: int, rank: int = 64, decay: float = 1.5,
                 noise_rel: float = 1e-3) -> np.ndarray:
    """Ill-conditioned momentum: U diag(i^-decay) V^T plus noise N with
    ||N||_F = noise_rel * ||U S V^T||_F.  U, V orthonormal (QR of Gaussians)."""
    rng = np.random.default_rng(seed)
    r = min(rank, n, m)
    u, _ = np.linalg.qr(rng.standard_normal((n, r)))
    v, _ = np.linalg.qr(rng.standard_normal((m, r)))
    sv = np.arange(1, r + 1, dtype=np.float64) ** (-decay)
    low = (u * sv) @ v.T
    noise = rng.standard_normal((n, m))
    noise *= noise_rel * np.linalg.norm(low) / np.linalg.norm(noise)
    return (low + noise).astype(np.float32)


def host_tied(n: int, m: int, seed: int, n_distinct: int) -> np.ndarray:
    """Matrix whose rows are sign-flipped, permuted copies of ``n_distinct``
    base rows with entries in {-2, -1.75, ..., 2}: every sum of their absolute
    values is exact in any order, so rows from one base row tie exactly in
    l1 (a tie-stress input)."""
    rng = np.random.default_rng(seed)
    base = (rng.integers(-8, 9, size=(n_distinct, m)) / 4.0).astype(np.float32)
    pick = rng.integers(0, n_distinct, size=n)
    out = np.empty((n, m), np.float32)
    for i in range(n):
        out[i] = rng.permutation(base[pick[i]]) * rng.choice(np.array([-1.0, 1.0], np.float32), size=m)
    return out


# -------------------------------------------------------------- device side

def device_matrix(kind: str, n: int, m: int, seed: int, device: str = "cuda"):
    """Draw one fp32 momentum matrix on the device (torch.Generator seeded)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    if kind == "gaussian":
        return torch.randn((n, m), generator=g, device=device, dtype=torch.float32)
    if kind == "scaled":
        x = torch.randn((n, m), generator=g, device=device, dtype=torch.float32)
        scale = 0.1 + 9.9 * torch.rand((), generator=g, device=device, dtype=torch.float64).item()
        return x.mul_(scale)
    if kind == "lowrank":
        # orthonormal factors from a host QR (seeded PCG64), product on the device
        rng = np.random.default_rng(seed)
        r = min(64, n, m)
        u, _ = np.linalg.qr(rng.standard_normal((n, r)))
        v, _ = np.linalg.qr(rng.standard_normal((m, r)))
        sv = np.arange(1, r + 1, dtype=np.float64) ** (-1.5)
        ud = torch.from_numpy((u * sv).astype(np.float32)).to(device)
        vd = torch.from_numpy(v.astype(np.float32)).to(device)
        low = ud @ vd.T
        noise = torch.randn((n, m), generator=g, device=device, dtype=torch.float32)
        noise.mul_(1e-3 * low.norm() / noise.norm())
        return low.add_(noise)
    raise ValueError(kind)


def device_weight(n: int, m: int, seed: int, device: str = "cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn((n, m), generator=g, device=device, dtype=torch.float32).mul_(W_STD)


def device_workload(wl: Workload, device: str = "cuda", groups: Optional[Sequence[int]] = None,
                    limit_per_group: Optional[int] = None):
    """Return ``[(group, [W_i], [M_i])]`` with every matrix on the device.

    Matrix ``i`` (running index over the whole set) draws M with seed
    ``seed_base + i`` and W with seed ``seed_base + 100000 + i``.
    """
    out = []
    idx = 0
    for gi, g in enumerate(wl.groups):
        ws: List = []
        ms: List = []
        for j in range(g.count):
            take = (groups is None or gi in groups) and (limit_per_group is None or j < limit_per_group)
            if take:
                ms.append(device_matrix(wl.kind, g.n, g.m, wl.seed_base + idx, device))
                ws.append(device_weight(g.n, g.m, wl.seed_base + 100000 + idx, device))
            idx += 1
        if ms:
            out.append((g, ws, ms))
    return out

