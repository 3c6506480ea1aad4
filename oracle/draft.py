"""Draft estimation and the shared ranking.

[DA2] abstract: spatially 2D average-pooled and max-pooled queries and keys
give complementary regional statistics; a low-resolution draft attention map
built from them estimates each block's importance; one ranking per query
block gives the top blocks the higher precision, the next retained blocks the
lower precision, and skips the rest, under configurable budgets.
[DA1] abstract: the draft map is attention between the down-sampled queries
and keys, over all frames. [DA1-article] steps 1-3: average pooling, draft
map, highest-scoring regions become the mask.

Readings (the pages give no formula):
* Pooling is over the window's real tokens only: channel-wise mean and
  channel-wise (signed) maximum.
* Each pooled pair gives a row-softmax map over all key blocks,
  A = softmax_rows(tau * Qp Kp^T), with the attention's own scale tau; the
  block score is the mean of the two maps, C = (A_avg + A_max) / 2, which is
  row-stochastic like a block attention mass.
* Counts per row: n_hi = floor(b_hi n_b + 1/2), n_ret = floor((b_hi + b_lo')
  n_b + 1/2) with b_lo' = min(b_lo, 1 - b_hi), n_lo = n_ret - n_hi, all in
  IEEE double, evaluated as written (no fused multiply-add). n_ret = 0 is an
  invalid configuration.
* Ranking order: C descending, ties to the lower block index.
"""

from __future__ import annotations

import math

import numpy as np

SKIP, LO, HI = 0, 1, 2


def pool_blocks(xb: np.ndarray, valid: np.ndarray):
    """xb [n_b, bs, d] float64 (padded slots arbitrary), valid [n_b, bs] bool -> (mean, max) [n_b, d]."""
    cnt = valid.sum(axis=1)
    s = np.where(valid[..., None], xb, 0.0).sum(axis=1)
    mean = s / cnt[:, None]
    mx = np.where(valid[..., None], xb, -np.inf).max(axis=1)
    return mean, mx


def _row_softmax(z: np.ndarray) -> np.ndarray:
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=1, keepdims=True)


def draft_scores(q_avg, q_max, k_avg, k_max, tau: float) -> np.ndarray:
    """C [n_b, n_b]: mean of the average-pooled and max-pooled draft maps."""
    a_avg = _row_softmax(tau * (q_avg @ k_avg.T))
    a_max = _row_softmax(tau * (q_max @ k_max.T))
    return 0.5 * (a_avg + a_max)


def budget_counts(n_blocks: int, budget_hi: float, budget_lo: float):
    """(n_hi, n_lo) per query block."""
    if budget_hi < 0 or budget_lo < 0 or budget_hi > 1:
        raise ValueError("budgets must lie in [0, 1]")
    lo = min(budget_lo, 1.0 - budget_hi)
    n_hi = math.floor(budget_hi * n_blocks + 0.5)
    n_ret = math.floor((budget_hi + lo) * n_blocks + 0.5)
    if n_ret < 1:
        raise ValueError("budgets retain no block")
    return n_hi, n_ret - n_hi


def rank_labels(C: np.ndarray, n_hi: int, n_lo: int) -> np.ndarray:
    """labels [n_b, n_b] int8: HI for ranks < n_hi, LO for the next n_lo, SKIP otherwise."""
    labels = np.zeros(C.shape, dtype=np.int8)
    j = np.arange(C.shape[1])
    for i in range(C.shape[0]):
        order = np.lexsort((j, -C[i]))          # primary: C descending; then index ascending
        labels[i, order[:n_hi]] = HI
        labels[i, order[n_hi:n_hi + n_lo]] = LO
    return labels


def exemption_mask(C: np.ndarray, n_hi: int, n_lo: int, rel: float = 1e-5) -> np.ndarray:
    """[n_b, n_b] bool: blocks whose score lies within rel of a budget threshold.

    The threshold t_k is the midpoint of the scores at ranks n_k and n_k + 1
    (k in {hi, retained}); such a block may carry either adjacent label.
    """
    nb = C.shape[1]
    out = np.zeros_like(C, dtype=bool)
    j = np.arange(nb)
    for i in range(C.shape[0]):
        order = np.lexsort((j, -C[i]))
        s = C[i, order]
        for n in (n_hi, n_hi + n_lo):
            if 0 < n < nb:
                t = 0.5 * (s[n - 1] + s[n])
                out[i] |= np.abs(C[i] - t) <= rel * t
    return out
