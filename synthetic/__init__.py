"""Seeded synthetic video-latent Q/K/V inputs.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic. Both the CPU oracle and the GPU path read the tensors it
returns, byte for byte.

Recipe (one generator, seeded, CPU, so the bytes are the same on every host):

* Q and K are smooth fields plus noise: for every (batch, head, frame, channel)
  a coarse grid of N(0, 1) values is upsampled bilinearly (half-pixel centres,
  i.e. ``align_corners=False``) by an integer factor, cropped to the latent
  grid, and N(0, sigma_noise^2) noise is added per token. Q and K use
  independent fields.
* V is N(0, 1) per element.
* ``outlier_channels`` channels (the same indices for Q and K, drawn from a
  seeded permutation) are multiplied by ``outlier_scale``.
* ``temporal_rho`` > 0 makes the coarse field an AR(1) process across frames:
  g_t = rho * g_{t-1} + sqrt(1 - rho^2) * eps_t.
* Layout is [B, H, N, d], N in raster order (frame, row, column), bf16.

The DraftAttention2 and DraftAttention pages evaluate on HunyuanVideo and
Wan2.1 activations, which are not available here; these fields stand in for
them with the same token-grid shapes.
"""

from __future__ import annotations

import dataclasses
import math

import torch
import torch.nn.functional as F


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    frames: int
    grid_h: int
    grid_w: int
    head_dim: int
    win_h: int
    win_w: int
    budget_hi: float
    budget_lo: float
    upsample: int
    noise_std: float = 0.3
    outlier_channels: int = 0
    outlier_scale: float = 8.0
    temporal_rho: float = 0.0
    seed: int = 0
    pack_edges: bool = False           # packed edge windows (geometry only; inputs unchanged)

    @property
    def tokens(self) -> int:
        return self.frames * self.grid_h * self.grid_w


TINY = Workload("tiny", 1, 1, 2, 16, 16, 64, 4, 4, 0.25, 0.25, upsample=4)
SMALL = Workload("small", 1, 2, 5, 32, 32, 128, 8, 16, 0.10, 0.30, upsample=8,
                 outlier_channels=2)
WAN480 = Workload("wan480p", 1, 12, 21, 30, 52, 128, 8, 16, 0.15, 0.35, upsample=8)
HUNYUAN720 = Workload("hunyuan720p", 1, 24, 33, 45, 80, 128, 8, 16, 0.10, 0.20,
                      upsample=8, temporal_rho=0.9)

WORKLOADS = {w.name: w for w in (TINY, SMALL, WAN480, HUNYUAN720)}

# Budget sweep on the Wan-480p shape: (hi, lo) fractions; the rest is skipped.
SWEEP_POINTS = [(h, l) for h in (0.05, 0.10, 0.25, 1.0) for l in (0.0, 0.2, 0.4)] + [(0.0, 1.0)]


def with_budgets(w: Workload, hi: float, lo: float) -> Workload:
    return dataclasses.replace(w, name=f"{w.name}-hi{hi:g}-lo{lo:g}", budget_hi=hi, budget_lo=lo)


def _smooth_field(gen: torch.Generator, w: Workload, batch: int, heads: int) -> torch.Tensor:
    """[B, H, T, Hl, Wl, d] float32 smooth field + noise."""
    f = w.upsample
    ch = -(-w.grid_h // f)
    cw = -(-w.grid_w // f)
    d = w.head_dim
    coarse = torch.randn(batch, heads, w.frames, d, ch, cw, generator=gen)
    if w.temporal_rho > 0.0:
        rho = w.temporal_rho
        innov = math.sqrt(1.0 - rho * rho)
        for t in range(1, w.frames):
            coarse[:, :, t] = rho * coarse[:, :, t - 1] + innov * coarse[:, :, t]
    flat = coarse.reshape(batch * heads * w.frames, d, ch, cw)
    up = F.interpolate(flat, size=(ch * f, cw * f), mode="bilinear", align_corners=False)
    up = up[:, :, : w.grid_h, : w.grid_w]
    up = up.reshape(batch, heads, w.frames, d, w.grid_h, w.grid_w).permute(0, 1, 2, 4, 5, 3)
    noise = torch.randn(up.shape, generator=gen) * w.noise_std
    return up + noise


def make_qkv(w: Workload):
    """Return (q, k, v) bf16 CPU tensors [B, H, N, d] for workload ``w``."""
    heads = w.heads
    gen = torch.Generator(device="cpu").manual_seed(w.seed)
    n = w.tokens
    d = w.head_dim
    q = _smooth_field(gen, w, w.batch, heads)
    k = _smooth_field(gen, w, w.batch, heads)
    if w.outlier_channels > 0:
        idx = torch.randperm(d, generator=gen)[: w.outlier_channels]
        q[..., idx] *= w.outlier_scale
        k[..., idx] *= w.outlier_scale
    v = torch.randn(w.batch, heads, n, d, generator=gen)
    q = q.reshape(w.batch, heads, n, d).to(torch.bfloat16).contiguous()
    k = k.reshape(w.batch, heads, n, d).to(torch.bfloat16).contiguous()
    v = v.to(torch.bfloat16).contiguous()
    return q, k, v
