"""Seeded synthetic workloads shared by the GPU path's tests/bench and the oracle.

This module holds no arithmetic of the method: it only draws random tensors
(torch's CPU generator, float32 normal draws, optional rounding to bf16) in a
fixed order so that both sides see the same bytes.

The pages measure on random Gaussian tensors ("AdaSplash: Adaptive Sparse Flash
Attention", measured-effects table: random tensors, n = 8192; "AdaSplash-2:
Faster Differentiable Sparse Attention", sec. 4.2: Gaussian Q/K/V, d = 64,
bf16, and sec. 4.1: Gaussian score vectors).  The named configurations below
stand in for those workloads; no dataset is used.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

MASK_NONE, MASK_CAUSAL, MASK_WINDOW_SINK = 0, 1, 2


@dataclass(frozen=True)
class AttnConfig:
    name: str
    B: int
    H: int
    L: int
    d: int
    dtype: str          # "f32" or "bf16" (Q, K, V and dO)
    mask: int
    window: int
    seed: int
    clusters: int = 0   # > 0: clustered Q/K (contiguous runs per centroid)
    with_grad: bool = False
    q_std: float = 1.0  # standard deviation of Q in plain mode

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


@dataclass(frozen=True)
class RowsConfig:
    name: str
    rows: int
    cols: int
    seed: int


# The five workloads (C3 runs in two mask modes on one input set).
C1 = AttnConfig("c1_L256_d64_f32", 1, 1, 256, 64, "f32", MASK_NONE, 0, seed=1)
C2 = RowsConfig("c2_rows8192x8192_f32", 8192, 8192, seed=2)
C3A = AttnConfig("c3a_B8H12L1024d64_causal", 8, 12, 1024, 64, "bf16", MASK_CAUSAL, 0, seed=3)
C3B = AttnConfig("c3b_B8H12L1024d64_window32_sink", 8, 12, 1024, 64, "bf16",
                 MASK_WINDOW_SINK, 32, seed=3)
C4 = AttnConfig("c4_B1H12L8192d64_clustered", 1, 12, 8192, 64, "bf16", MASK_NONE, 0,
                seed=4, clusters=64)
C5 = AttnConfig("c5_B1H16L16384d128_causal_fwdbwd", 1, 16, 16384, 128, "bf16",
                MASK_CAUSAL, 0, seed=5, with_grad=True)

CONFIGS = {c.name: c for c in (C1, C2, C3A, C3B, C4, C5)}


def _round(t: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t
    raise ValueError(dtype)


def gen_rows(rows: int, cols: int, seed: int) -> torch.Tensor:
    """fp32 score matrix with i.i.d. N(0, 1) entries."""
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(rows, cols, generator=g, dtype=torch.float32)


def gen_attn(B: int, H: int, L: int, d: int, dtype: str, seed: int,
             clusters: int = 0, with_grad: bool = False,
             q_std: float = 1.0) -> dict:
    """Q, K, V (and dO) of shape [B, H, L, d] on the CPU.

    Plain mode: Q, K, V, dO i.i.d. N(0, 1) (Q scaled by q_std), drawn in that
    order.  Clustered mode (clusters = n_c > 0): per (b, h) n_c centroids
    3*N(0, 1) in R^d; position r uses centroid floor(r * n_c / L) (contiguous
    runs of L / n_c positions); Q = centroid + 0.3*N(0, 1), K = centroid +
    independent 0.3*N(0, 1), V = N(0, 1).  Draw order: centroids, Q noise,
    K noise, V, dO.
    """
    g = torch.Generator("cpu").manual_seed(seed)
    shape = (B, H, L, d)
    if clusters > 0:
        cent = 3.0 * torch.randn(B, H, clusters, d, generator=g, dtype=torch.float32)
        idx = (torch.arange(L) * clusters) // L
        base = cent[:, :, idx, :]
        q = base + 0.3 * torch.randn(shape, generator=g, dtype=torch.float32)
        k = base + 0.3 * torch.randn(shape, generator=g, dtype=torch.float32)
        v = torch.randn(shape, generator=g, dtype=torch.float32)
    else:
        q = q_std * torch.randn(shape, generator=g, dtype=torch.float32)
        k = torch.randn(shape, generator=g, dtype=torch.float32)
        v = torch.randn(shape, generator=g, dtype=torch.float32)
    out = {"q": _round(q, dtype), "k": _round(k, dtype), "v": _round(v, dtype)}
    if with_grad:
        out["do"] = _round(torch.randn(shape, generator=g, dtype=torch.float32), dtype)
    return out


def gen_config(cfg: AttnConfig, L: Optional[int] = None, H: Optional[int] = None,
               B: Optional[int] = None) -> dict:
    """Inputs of a named attention config, optionally at a smaller B/H/L."""
    return gen_attn(B or cfg.B, H or cfg.H, L or cfg.L, cfg.d, cfg.dtype, cfg.seed,
                    clusters=cfg.clusters, with_grad=cfg.with_grad, q_std=cfg.q_std)


def sweep_configs() -> list[AttnConfig]:
    """Block-sparsity sweep: the C4 generator with fewer, longer cluster runs."""
    out = []
    for i, nc in enumerate((64, 32, 16, 8, 4, 2, 1)):
        out.append(AttnConfig(f"sweep_nc{nc}", 1, 12, 8192, 64, "bf16", MASK_NONE, 0,
                              seed=40 + i, clusters=nc))
    return out


QVAR_STDS = (0.1, 0.25, 0.5, 1.0, 2.0, 4.0, 8.0, 16.0, 32.0)


def qvar_configs() -> list[AttnConfig]:
    """Query-variance sweep ("AdaSplash-2: Faster Differentiable Sparse
    Attention", sec. 4.2: Gaussian Q/K/V, d = 64, bf16, block sparsity set by
    the variance of the queries): B1 H12 L8192 d64, K and V ~ N(0, 1),
    Q ~ N(0, s^2) for each s of QVAR_STDS, scale 1/8, no mask.  Small s gives
    near-uniform rows with supports of hundreds of keys, large s near one-hot
    rows."""
    return [AttnConfig(f"qvar_std{sd:g}", 1, 12, 8192, 64, "bf16", MASK_NONE, 0, seed=50 + i, q_std=sd)
            for i, sd in enumerate(QVAR_STDS)]
