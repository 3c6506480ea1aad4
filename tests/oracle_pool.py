"""The oracle's attention over many query blocks, in a pool of CPU processes.

Test infrastructure. The workers are spawned, not forked, so they inherit no
GPU state and never touch the GPU: each one rebuilds the oracle's per-head
state from that head's bf16 input bytes (the same bytes the GPU read) and
computes a share of the query blocks with one BLAS thread. Nothing computed
on the GPU reaches a worker.
"""

from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os
import types

import numpy as np

_STATE = None


def pool_size() -> int:
    """Worker count: the CPUs this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _init(cfg: dict, q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray):
    global _STATE
    from threadpoolctl import threadpool_limits

    from oracle import pipeline as P
    threadpool_limits(limits=1)
    ns = types.SimpleNamespace(**cfg)
    _STATE = P.prepare_head(ns, _bf16_bits_to_f64(q_bits), _bf16_bits_to_f64(k_bits), _bf16_bits_to_f64(v_bits))


def _rows(blocks):
    from oracle import pipeline as P
    st = _STATE
    out = P.attention_raster(st, blocks=blocks)
    rows = np.concatenate([st.idx[i][st.valid[i]] for i in blocks])
    return rows, out[rows]


def workload_dict(w) -> dict:
    """The fields of a workload the oracle reads."""
    keys = ("name", "frames", "grid_h", "grid_w", "head_dim", "win_h", "win_w", "budget_hi", "budget_lo",
            "pack_edges")
    d = {k: getattr(w, k) for k in keys}
    d["softmax_scale"] = getattr(w, "softmax_scale", 0.0)
    return d


def attention_rows(w, q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, blocks, workers=None):
    """Oracle outputs of one (batch, head) for the real rows of the given
    query blocks: (raster row indices, float64 [rows, d]).

    q_bits, k_bits, v_bits: uint16 [N, d], the head's bf16 bit patterns."""
    blocks = [int(b) for b in blocks]
    n = workers or pool_size()
    n = max(1, min(n, len(blocks)))
    chunks = [blocks[i::n] for i in range(n)]
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(max_workers=n, mp_context=ctx, initializer=_init,
                                initargs=(workload_dict(w), q_bits, k_bits, v_bits)) as ex:
        parts = list(ex.map(_rows, chunks))
    rows = np.concatenate([p[0] for p in parts])
    vals = np.concatenate([p[1] for p in parts])
    order = np.argsort(rows, kind="stable")
    return rows[order], vals[order]
