"""Error decomposition and draft-map fidelity (diagnostics, float64).

TEST INFRASTRUCTURE ONLY, like the rest of this package: these functions
measure the method on small inputs; nothing on the product path calls them.

[DA2] "DraftAttention2" (arXiv 2609.32628), abstract: two terms make up the
method's output error, one from the blocks it drops (sparsification) and one
from the blocks it keeps at reduced precision, weighted by their attention
(quantization). Moving a block from "skipped" to "4-bit" trades the first
for the second, so it pays off whenever the block's rounding error is the
smaller of the two; hence many blocks kept at low precision and the highest
precision reserved for the blocks with the most attention mass.
[DA1-article] (the news write-up of DraftAttention), theory paragraph: the
draft map built from pooled queries and keys stays close to the full-
resolution map in Frobenius norm, closer for spatially smooth latents, and
the error of the sparse mask taken from it is bounded.

Readings (the pages print no formula):
* Sparsification error: O_sparse - O_dense, where O_sparse is exact
  (unquantized) softmax attention over the retained blocks' keys only and
  O_dense is softmax attention over all keys.
* Quantization error: O_method - O_sparse (same retained blocks, the
  method's operands and P quantization).
* Block attention mass M[i, j]: the mean, over the real query tokens of block
  i, of the dense attention probability on the real keys of block j (rows
  sum to one, like the draft score C).
* Draft-map error: ||C - M||_F / ||M||_F.
"""

from __future__ import annotations

import numpy as np

from .draft import HI, LO
from .pipeline import HeadState, attention_raster, dense_attention


def dense_probabilities(q: np.ndarray, k: np.ndarray, tau: float, rows=None) -> np.ndarray:
    """softmax_rows(tau Q K^T) in float64 for the given query rows (default all)."""
    qq = q if rows is None else q[rows]
    s = tau * (qq @ k.T)
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=1, keepdims=True)


def true_block_mass(st: HeadState, q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """M [n_b, n_b]: mean over block i's real query tokens of the dense
    attention mass on block j's real keys."""
    nb = st.geo.n_blocks
    P = dense_probabilities(q, k, st.tau)                  # [N, N] raster order
    M = np.zeros((nb, nb))
    key_cols = [st.idx[j][st.valid[j]] for j in range(nb)]
    for i in range(nb):
        rows = st.idx[i][st.valid[i]]
        Pi = P[rows]
        M[i] = [Pi[:, cols].sum(axis=1).mean() for cols in key_cols]
    return M


def _rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def error_split(st: HeadState, q: np.ndarray, k: np.ndarray, v: np.ndarray, labels=None) -> dict:
    """Relative L2 errors over all real rows: total (method vs dense),
    sparsification (exact sparse vs dense) and quantization (method vs exact
    sparse), plus the three outputs."""
    dense = dense_attention(q, k, v, st.tau)
    sparse = attention_raster(st, labels=labels, quantize=False)
    method = attention_raster(st, labels=labels, quantize=True)
    return {
        "total": _rel_l2(method, dense),
        "sparsification": _rel_l2(sparse, dense),
        "quantization": _rel_l2(method, sparse),
        "quantization_rel_to_dense": float(np.linalg.norm(method - sparse) / np.linalg.norm(dense)),
        "dense": dense,
        "sparse": sparse,
        "method": method,
    }


def mass_stats(M: np.ndarray, labels: np.ndarray) -> dict:
    """Per query block: the true mass of its hi, lo and retained blocks, the
    most mass any selection of the same size could retain, and their ratio
    (retained-mass recall), averaged over query blocks."""
    hi = np.where(labels == HI, M, 0.0).sum(axis=1)
    lo = np.where(labels == LO, M, 0.0).sum(axis=1)
    n_ret = (labels != 0).sum(axis=1)
    best = np.array([np.sort(row)[::-1][:n].sum() for row, n in zip(M, n_ret)])
    return {
        "hi_mass": float(hi.mean()),
        "lo_mass": float(lo.mean()),
        "retained_mass": float((hi + lo).mean()),
        "best_mass": float(best.mean()),
        "recall": float(((hi + lo) / best).mean()),
    }


def draft_map_error(C: np.ndarray, M: np.ndarray) -> float:
    """Relative Frobenius distance between the draft score map and the true
    block attention mass."""
    return float(np.linalg.norm(C - M) / np.linalg.norm(M))
