"""The whole path for one (batch, head): geometry, pool, draft map, rank,
quantize, attention, restore to raster order; plus dense attention for error
reporting.

Inputs are float64 arrays holding the bf16 values exactly (the caller upcasts).
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

from .attention import attend_block
from .draft import budget_counts, draft_scores, pool_blocks, rank_labels
from .geometry import Geometry, gather_blocks
from .quant import prepare_operands


def softmax_scale(cfg) -> float:
    s = getattr(cfg, "softmax_scale", 0.0) or 0.0
    return s if s > 0 else 1.0 / math.sqrt(cfg.head_dim)


@dataclasses.dataclass
class HeadState:
    geo: Geometry
    idx: np.ndarray          # [n_b, bs] raster index or -1
    valid: np.ndarray        # [n_b, bs] bool
    q_avg: np.ndarray
    q_max: np.ndarray
    k_avg: np.ndarray
    k_max: np.ndarray
    scores: np.ndarray       # C [n_b, n_b]
    n_hi: int
    n_lo: int
    labels: np.ndarray       # [n_b, n_b] int8
    ops: dict
    tau: float


def prepare_head(cfg, q: np.ndarray, k: np.ndarray, v: np.ndarray) -> HeadState:
    """q, k, v [N, d] float64 of one (batch, head)."""
    geo = Geometry(cfg.frames, cfg.grid_h, cfg.grid_w, cfg.win_h, cfg.win_w,
                   pack_edges=bool(getattr(cfg, "pack_edges", False)))
    idx = geo.raster_index()
    valid = idx >= 0
    qb, kb, vb = (gather_blocks(t, idx) for t in (q, k, v))
    q_avg, q_max = pool_blocks(qb, valid)
    k_avg, k_max = pool_blocks(kb, valid)
    tau = softmax_scale(cfg)
    C = draft_scores(q_avg, q_max, k_avg, k_max, tau)
    n_hi, n_lo = budget_counts(geo.n_blocks, cfg.budget_hi, cfg.budget_lo)
    labels = rank_labels(C, n_hi, n_lo)
    ops = prepare_operands(qb, kb, vb)
    ops.update(q=qb, k=kb, v=vb)
    return HeadState(geo, idx, valid, q_avg, q_max, k_avg, k_max, C, n_hi, n_lo, labels, ops, tau)


def attention_raster(st: HeadState, blocks=None, labels=None, quantize: bool = True) -> np.ndarray:
    """O [N, d] in raster order for the query blocks in ``blocks`` (default all);
    rows of other blocks are NaN. ``labels`` overrides the ranking's labels."""
    labels = st.labels if labels is None else labels
    n, d = st.geo.tokens, st.ops["q"].shape[-1]
    out = np.full((n, d), np.nan)
    for i in (range(st.geo.n_blocks) if blocks is None else blocks):
        ob = attend_block(i, labels[i], st.ops, st.valid, st.tau, quantize=quantize)
        sel = st.valid[i]
        out[st.idx[i][sel]] = ob[sel]
    return out


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, tau: float, rows=None) -> np.ndarray:
    """Textbook softmax(tau Q K^T) V in float64 over all tokens (for error reporting)."""
    qq = q if rows is None else q[rows]
    s = tau * (qq @ k.T)
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p @ v) / p.sum(axis=1, keepdims=True)
