"""Shared helpers for the GPU parity tests: run the library through the C ABI on
seeded synthetic inputs and compare against the CPU oracle.

Nothing here feeds a GPU result into the oracle: the oracle sees only the
generator's bf16 bytes and its own labels.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import synthetic as S
from oracle import draft as D
from oracle import formats as F
from oracle import pipeline as P

OUT_TOL = 2e-3          # max-abs output tolerance vs the oracle (same quantized operands)


def say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def np64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


class GpuRun:
    """Inputs on the device, a plan and a workspace after da2_prepare."""

    def __init__(self, da2, w: S.Workload, out_fp32: bool = True, qkv=None):
        self.da2 = da2
        self.w = w
        self.qc, self.kc, self.vc = S.make_qkv(w) if qkv is None else qkv
        self.q, self.k, self.v = (t.cuda() for t in (self.qc, self.kc, self.vc))
        cfg = da2.make_config(w.batch, w.heads, w.frames, w.grid_h, w.grid_w, w.head_dim, w.win_h, w.win_w,
                              w.budget_hi, w.budget_lo,
                              out_dtype=da2.DA2_OUT_FP32 if out_fp32 else da2.DA2_OUT_BF16,
                              flags=da2.DA2_FLAG_PACK_EDGES if w.pack_edges else 0)
        self.plan = da2.da2_plan(cfg)
        self.info = self.plan.info
        self.nb = self.info.n_blocks
        self.bh = w.batch * w.heads
        self.ws = self.plan.workspace()
        say(f"da2_prepare {w.name} B={w.batch} H={w.heads} N={w.tokens} d={w.head_dim} nb={self.nb} pack={int(w.pack_edges)} "
            f"n_hi={self.info.n_hi} n_lo={self.info.n_lo}")
        da2.da2_prepare(self.plan, self.q, self.k, self.v, self.ws)
        torch.cuda.synchronize()

    def sec(self, name, dtype, shape) -> np.ndarray:
        return self.da2.workspace_section(self.plan, self.ws, name, dtype, shape).cpu().numpy()

    def attend(self, out_fp32=True) -> torch.Tensor:
        w = self.w
        out = torch.full((w.batch, w.heads, w.tokens, w.head_dim), float("nan"),
                         dtype=torch.float32 if out_fp32 else torch.bfloat16, device="cuda")
        say(f"da2_attention {w.name}")
        self.da2.da2_attention(self.plan, self.ws, out)
        torch.cuda.synchronize()
        return out

    def set_labels(self, labels: np.ndarray) -> int:
        lab = torch.from_numpy(np.ascontiguousarray(labels.astype(np.int8))).cuda()
        say(f"da2_set_labels {self.w.name}")
        self.da2.da2_set_labels(self.plan, self.ws, lab)
        torch.cuda.synchronize()
        return int(self.sec("status", torch.int32, (4,))[0])

    def oracle_head(self, bh: int) -> P.HeadState:
        b, h = divmod(bh, self.w.heads)
        return P.prepare_head(self.w, np64(self.qc[b, h]), np64(self.kc[b, h]), np64(self.vc[b, h]))


def check_prepare(run: GpuRun, bh: int, st: P.HeadState):
    """Codes, scales, pooled values, scores, labels and lists of one (batch, head)."""
    w, nb, BH = run.w, run.nb, run.bh
    bs, d = st.geo.block_size, w.head_dim
    T = 128
    e8 = run.sec("e8", torch.uint8, (3, BH, nb)).astype(int) - 127
    for t, name in enumerate(("q", "k", "v")):
        assert np.array_equal(e8[t, bh], st.ops[name + "8_exp"]), f"{name} fp8 scale"
    for name in ("q", "k"):
        c8 = run.sec(name + "8", torch.uint8, (BH, nb, T, T))[bh]
        assert np.array_equal(c8[:, :bs, :d], st.ops[name + "8"]), f"{name} fp8 codes"
        assert not c8[:, bs:, :].any() and not c8[:, :, d:].any()
        c4 = unpack_nibbles(run.sec(name + "4", torch.uint8, (BH, nb, T, T // 2))[bh])
        assert np.array_equal(c4[:, :bs, :d], st.ops[name + "4"]), f"{name} mxfp4 codes"
        s4 = run.sec("s" + name + "4", torch.uint8, (BH, nb, T, 4))[bh].astype(int) - 127
        assert np.array_equal(s4[:, :bs, : d // 32], st.ops[name + "4_exp"]), f"{name} mxfp4 scales"
    v8 = run.sec("v8t", torch.uint8, (BH, nb, T, T))[bh]
    assert np.array_equal(v8[:, :d, :bs], np.swapaxes(st.ops["v8"], 1, 2)), "v fp8 codes"
    v4 = unpack_nibbles(run.sec("v4t", torch.uint8, (BH, nb, T, T // 2))[bh])
    assert np.array_equal(v4[:, :d, :bs], st.ops["v4t"]), "v mxfp4 codes"
    G = st.ops["v4t_exp"].shape[-1]
    sv = run.sec("sv4t", torch.uint8, (BH, nb, T, 4))[bh].astype(int) - 127
    assert np.array_equal(sv[:, :d, :G], st.ops["v4t_exp"]), "v mxfp4 scales"
    # key-slot bias: 0 for a token, -inf for a padded slot, and a last row for
    # the empty key tile (every slot -inf)
    bias = run.sec("bias", torch.float32, (nb + 1, T))
    want_bias = np.full((nb + 1, T), -np.inf, dtype=np.float32)
    for i in range(nb):
        want_bias[i, :bs][st.valid[i]] = 0.0
    assert np.array_equal(bias, want_bias), "key-slot bias"
    pool = run.sec("pool", torch.float64, (4, BH, nb, T))[:, bh, :, :d]
    np.testing.assert_allclose(pool[0], st.q_avg, rtol=1e-14, atol=1e-300)
    np.testing.assert_array_equal(pool[1], st.q_max)
    np.testing.assert_allclose(pool[2], st.k_avg, rtol=1e-14, atol=1e-300)
    np.testing.assert_array_equal(pool[3], st.k_max)
    C = run.sec("scores", torch.float64, (2, BH, nb, nb))[0, bh]
    np.testing.assert_allclose(C, st.scores, rtol=1e-10, atol=1e-300)
    lab = run.sec("labels", torch.int8, (BH, nb, nb))[bh]
    n_hi, n_lo = st.n_hi, st.n_lo
    assert np.all((lab == D.HI).sum(1) == n_hi) and np.all((lab == D.LO).sum(1) == n_lo)
    diff = lab != st.labels
    if diff.any():
        ex = D.exemption_mask(st.scores, n_hi, n_lo)
        assert not (diff & ~ex).any(), "labels differ outside the exemption band"
    # every row also follows the ranking rule on the GPU's own C (C
    # descending, lower index first), which decides what the band leaves
    # open: rows of exactly equal scores, for one
    order = np.lexsort((np.broadcast_to(np.arange(nb), C.shape), -C), axis=-1)
    ranked = np.full((nb, nb), D.SKIP, dtype=np.int8)
    rows = np.arange(nb)[:, None]
    ranked[rows, order[:, :n_hi]] = D.HI
    ranked[rows, order[:, n_hi:n_hi + n_lo]] = D.LO
    assert np.array_equal(lab, ranked), "labels break the (C descending, index ascending) rule on the GPU's C"
    # lists: the labelled blocks in rank order (the GPU's own C descending, lower index first)
    for name, lv, n in (("hi", D.HI, n_hi), ("lo", D.LO, n_lo)):
        if not n:
            continue
        lst = run.sec(name, torch.int32, (BH, nb, n))[bh]
        for i in range(nb):
            members = np.flatnonzero(lab[i] == lv)
            want = sorted(members, key=lambda j: (-C[i, j], j))
            assert list(lst[i]) == want, f"{name} list of row {i}"
    return lab


def compare_outputs(got: np.ndarray, want: np.ndarray, rows: np.ndarray, tol: float = OUT_TOL):
    """Max-abs over the given raster rows; also reports how many rows exceed tol."""
    g, r = got[rows], want[rows]
    assert np.isfinite(g).all(), "non-finite output"
    err = np.abs(g - r).max(axis=1)
    worst = float(err.max()) if err.size else 0.0
    say(f"   rows={len(rows)} max|d|={worst:.3e} rows>tol={(err > tol).sum()}")
    return worst, int((err > tol).sum())


def block_rows(st: P.HeadState, blocks) -> np.ndarray:
    rows = [st.idx[i][st.valid[i]] for i in blocks]
    return np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)
