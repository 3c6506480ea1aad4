"""Pins for oracle.attention / oracle.pipeline: invariants, torch SDPA in float64,
hand-derived P quantization, single-key and constant-V closed forms, brute force."""

import json
import math
import os
from types import SimpleNamespace

import numpy as np
import pytest
import torch
import torch.nn.functional as TF

from oracle import attention as A
from oracle import draft as D
from oracle import pipeline as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cfg(frames=2, gh=8, gw=8, d=16, wh=4, ww=4, hi=0.25, lo=0.25):
    return SimpleNamespace(frames=frames, grid_h=gh, grid_w=gw, head_dim=d, win_h=wh, win_w=ww,
                           budget_hi=hi, budget_lo=lo, softmax_scale=0.0)


def _qkv(cfg, seed=0, vconst=None):
    rng = np.random.default_rng(seed)
    n = cfg.frames * cfg.grid_h * cfg.grid_w
    q = rng.normal(size=(n, cfg.head_dim)) * 1.5
    k = rng.normal(size=(n, cfg.head_dim)) * 1.5
    v = rng.normal(size=(n, cfg.head_dim)) if vconst is None else np.full((n, cfg.head_dim), vconst)
    return q, k, v


def test_p_quantization_hand_derived():
    g = json.load(open(os.path.join(GOLDEN, "p_quant_cases.json")))
    for case in g["hi"]:
        assert A.quantize_p_hi(np.array([case["p"]]))[0] == case["expect"], case
    for case in g["lo"]:
        p = np.zeros(32)
        p[: len(case["p"])] = case["p"]
        got = A.quantize_p_lo(p[None])[0]
        assert got[: len(case["p"])].tolist() == case["expect"], case
        assert np.all(got[len(case["p"]):] == 0)


def test_p_quantization_power_of_two_shift_invariance():
    rng = np.random.default_rng(7)
    p = rng.random((50, 128)) ** 3
    for k in (-9, -1, 3, 17):
        assert np.array_equal(A.quantize_p_lo(p * 2.0 ** k), A.quantize_p_lo(p) * 2.0 ** k)
    pn = p[p * 256 >= 2.0 ** -6 * 2 ** 5]      # stays in the normal range after the shift
    for k in (1, 3, 5):
        assert np.array_equal(A.quantize_p_hi(pn * 2.0 ** -k) * 2.0 ** k, A.quantize_p_hi(pn))


def test_constant_v_is_reproduced_exactly():
    cfg = _cfg(hi=0.25, lo=0.5)
    q, k, v = _qkv(cfg, vconst=1.5)          # 1.5 is exact in E4M3 and E2M1
    st = P.prepare_head(cfg, q, k, v)
    assert (st.labels == D.HI).any() and (st.labels == D.LO).any()
    O = P.attention_raster(st)
    assert np.all(O == 1.5)


def test_weights_sum_to_one_over_retained_blocks_only():
    cfg = _cfg(gh=10, gw=9, hi=0.25, lo=0.25)          # partial windows present
    q, k, v = _qkv(cfg, seed=1)
    st = P.prepare_head(cfg, q, k, v)
    for i in range(st.geo.n_blocks):
        _, w = A.attend_block(i, st.labels[i], st.ops, st.valid, st.tau, return_weights=True)
        rows = st.valid[i]
        np.testing.assert_allclose(w[rows].sum(axis=(1, 2)), 1.0, rtol=1e-14)
        assert np.all(w[:, st.labels[i] == D.SKIP] == 0)
        assert np.all(w[:, ~st.valid] == 0)
        assert np.all(w >= 0)


def _masked_sdpa(q, k, v, tau, mask):
    """torch reference: softmax(tau q k^T + (-inf off mask)) v in float64."""
    qt, kt, vt = (torch.from_numpy(x)[None, None] for x in (q, k, v))
    out = TF.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask)[None, None],
                                          scale=tau)
    return out[0, 0].numpy()


@pytest.mark.parametrize("pack", [False, True])
def test_unquantized_all_high_equals_dense_sdpa(pack):
    cfg = _cfg(frames=2, gh=9, gw=10, hi=1.0, lo=0.0)
    cfg.pack_edges = pack
    q, k, v = _qkv(cfg, seed=2)
    st = P.prepare_head(cfg, q, k, v)
    assert np.all(st.labels == D.HI)
    O = P.attention_raster(st, quantize=False)
    ref = _masked_sdpa(q, k, v, st.tau, np.ones((q.shape[0], q.shape[0]), dtype=bool))
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(P.dense_attention(q, k, v, st.tau), ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("pack", [False, True])
def test_unquantized_sparse_equals_block_masked_sdpa(pack):
    cfg = _cfg(frames=2, gh=9, gw=10, hi=0.2, lo=0.3)
    cfg.pack_edges = pack
    q, k, v = _qkv(cfg, seed=3)
    st = P.prepare_head(cfg, q, k, v)
    n = q.shape[0]
    block_of = np.empty(n, dtype=int)
    for b in range(st.geo.n_blocks):
        block_of[st.idx[b][st.valid[b]]] = b
    mask = st.labels[block_of][:, block_of] != D.SKIP          # [token, token]
    O = P.attention_raster(st, quantize=False)
    ref = _masked_sdpa(q, k, v, st.tau, mask)
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("phase", [D.HI, D.LO])
def test_single_retained_key_returns_its_value(phase):
    cfg = _cfg(frames=1, gh=5, gw=5, hi=0.25, lo=0.0)       # window 4x4: block 3 holds one token
    q, k, v = _qkv(cfg, seed=4)
    st = P.prepare_head(cfg, q, k, v)
    assert st.valid[3].sum() == 1
    labels = np.zeros_like(st.labels)
    labels[:, 3] = phase
    O = P.attention_raster(st, labels=labels)
    slot = int(np.flatnonzero(st.valid[3])[0])
    vq = st.ops["v8_deq" if phase == D.HI else "v4_deq"][3, slot]
    assert np.all(O == vq[None, :])


def _brute_force(cfg, q, k, v):
    """Pure-Python loops over the same definitions (tiny shapes only)."""
    from oracle.formats import decode_e2m1, decode_e4m3, encode_e2m1, encode_e4m3, shared_exponent
    st = P.prepare_head(cfg, q, k, v)
    ops, nb, bs = st.ops, st.geo.n_blocks, st.geo.block_size
    tau = 1.0 / math.sqrt(cfg.head_dim)
    out = np.full_like(q, np.nan)
    for i in range(nb):
        for s in range(bs):
            if not st.valid[i, s]:
                continue
            xs = {}
            for j in range(nb):
                lab = st.labels[i, j]
                if lab == D.SKIP:
                    continue
                qv = ops["q8_deq" if lab == D.HI else "q4_deq"][i, s]
                for t in range(bs):
                    if st.valid[j, t]:
                        kv = ops["k8_deq" if lab == D.HI else "k4_deq"][j, t]
                        xs[(j, t)] = sum(float(a) * float(b) for a, b in zip(qv, kv)) * tau / math.log(2)
            m = math.ceil(max(xs.values()))
            num = np.zeros(cfg.head_dim)
            den = 0.0
            for j in range(nb):
                lab = st.labels[i, j]
                if lab == D.SKIP:
                    continue
                ps = [2.0 ** (xs[(j, t)] - m) if (j, t) in xs else 0.0 for t in range(bs)]
                if lab == D.HI:
                    pq = [float(decode_e4m3(encode_e4m3([p * 256.0]))[0]) / 256.0 for p in ps]
                    vv = ops["v8_deq"][j]
                else:
                    pq = []
                    for g0 in range(0, bs, 32):
                        grp = ps[g0:g0 + 32]
                        e = int(shared_exponent(max(grp), 6.0))
                        pq += [float(decode_e2m1(encode_e2m1([p / 2.0 ** e]))[0]) * 2.0 ** e for p in grp]
                    vv = ops["v4_deq"][j]
                for t in range(bs):
                    num += pq[t] * vv[t]
                    den += pq[t]
            out[st.idx[i, s]] = num / den
    return out


def test_brute_force_micro_pipeline():
    cfg = _cfg(frames=2, gh=6, gw=7, d=16, hi=0.25, lo=0.375)
    q, k, v = _qkv(cfg, seed=6)
    st = P.prepare_head(cfg, q, k, v)
    np.testing.assert_allclose(P.attention_raster(st), _brute_force(cfg, q, k, v), rtol=0, atol=1e-12)
