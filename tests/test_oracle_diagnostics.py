"""Pins for oracle.diagnostics: the error split and the draft-fidelity measures.

Each pin reaches the quantity by a route the diagnostics code does not take
(attention with indicator values, piecewise-constant tokens whose block mass
has a closed form, selections built from the true mass) or checks a property
the definitions force (rows of a mass map sum to one, a full selection has no
sparsification error, the triangle inequality).
"""

from types import SimpleNamespace

import numpy as np
import pytest

from oracle import diagnostics as X
from oracle import draft as D
from oracle import pipeline as P
from oracle.geometry import Geometry


def _cfg(frames=2, gh=8, gw=8, d=16, wh=4, ww=4, hi=0.25, lo=0.25):
    return SimpleNamespace(frames=frames, grid_h=gh, grid_w=gw, head_dim=d, win_h=wh, win_w=ww,
                           budget_hi=hi, budget_lo=lo, softmax_scale=0.0)


def _qkv(cfg, seed=0, scale=1.5):
    rng = np.random.default_rng(seed)
    n = cfg.frames * cfg.grid_h * cfg.grid_w
    return (rng.normal(size=(n, cfg.head_dim)) * scale, rng.normal(size=(n, cfg.head_dim)) * scale,
            rng.normal(size=(n, cfg.head_dim)))


def _block_constant(cfg, seed=0, scale=1.5):
    """q and k constant over each window's tokens (v random)."""
    rng = np.random.default_rng(seed)
    n = cfg.frames * cfg.grid_h * cfg.grid_w
    st = P.prepare_head(cfg, *(np.zeros((n, cfg.head_dim)),) * 3)
    q, k = np.empty((n, cfg.head_dim)), np.empty((n, cfg.head_dim))
    for i in range(st.geo.n_blocks):
        rows = st.idx[i][st.valid[i]]
        q[rows] = rng.normal(size=cfg.head_dim) * scale
        k[rows] = rng.normal(size=cfg.head_dim) * scale
    return q, k, rng.normal(size=(n, cfg.head_dim))


def test_block_mass_equals_attention_of_block_indicators():
    # attending with V = one-hot block membership returns each row's mass per
    # key block; averaging over a block's rows gives M (ragged windows included)
    cfg = _cfg(gh=10, gw=9)
    q, k, v = _qkv(cfg, seed=3)
    st = P.prepare_head(cfg, q, k, v)
    nb, n = st.geo.n_blocks, st.geo.tokens
    onehot = np.zeros((n, nb))
    for j in range(nb):
        onehot[st.idx[j][st.valid[j]], j] = 1.0
    assert np.all(onehot.sum(axis=1) == 1)
    per_row = P.dense_attention(q, k, onehot, st.tau)
    want = np.stack([per_row[st.idx[i][st.valid[i]]].mean(axis=0) for i in range(nb)])
    M = X.true_block_mass(st, q, k)
    np.testing.assert_allclose(M, want, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(M.sum(axis=1), 1.0, rtol=1e-13)
    assert np.all(M > 0)


def test_block_constant_tokens_make_the_draft_map_exact():
    # with q and k constant over full windows, both pooled maps equal the
    # block-level softmax, which is also the exact block mass
    cfg = _cfg()
    q, k, v = _block_constant(cfg, seed=5)
    st = P.prepare_head(cfg, q, k, v)
    assert st.valid.all()
    M = X.true_block_mass(st, q, k)
    assert X.draft_map_error(st.scores, M) < 1e-12
    s = X.mass_stats(M, st.labels)
    assert s["recall"] == pytest.approx(1.0, abs=1e-12)


def test_full_retention_has_no_sparsification_error():
    cfg = _cfg(hi=1.0, lo=0.0)
    q, k, v = _qkv(cfg, seed=1)
    st = P.prepare_head(cfg, q, k, v)
    e = X.error_split(st, q, k, v)
    assert e["sparsification"] < 1e-13
    assert 0 < e["quantization"] < 0.1            # fp8 E4M3 operands and P
    assert e["total"] == pytest.approx(e["quantization"], rel=1e-9)
    s = X.mass_stats(X.true_block_mass(st, q, k), st.labels)
    assert s["retained_mass"] == pytest.approx(1.0, abs=1e-12)
    assert s["recall"] == pytest.approx(1.0, abs=1e-12)


def test_error_split_triangle_and_consistency():
    cfg = _cfg(gh=10, gw=9, hi=0.1, lo=0.3)
    q, k, v = _qkv(cfg, seed=2)
    st = P.prepare_head(cfg, q, k, v)
    e = X.error_split(st, q, k, v)
    assert np.isfinite(e["method"]).all() and np.isfinite(e["sparse"]).all()
    assert e["sparsification"] > 0 and e["quantization"] > 0
    assert e["total"] <= e["sparsification"] + e["quantization_rel_to_dense"] + 1e-12
    np.testing.assert_allclose(e["dense"], P.dense_attention(q, k, v, st.tau), rtol=0, atol=0)


def test_recall_of_mass_ranked_selection_is_one():
    cfg = _cfg(gh=10, gw=9)
    q, k, v = _qkv(cfg, seed=4)
    st = P.prepare_head(cfg, q, k, v)
    M = X.true_block_mass(st, q, k)
    ideal = D.rank_labels(M, st.n_hi, st.n_lo)
    s = X.mass_stats(M, ideal)
    assert s["recall"] == pytest.approx(1.0, abs=1e-12)
    assert s["retained_mass"] == pytest.approx(s["best_mass"], abs=1e-12)
    # the reversed ranking keeps the least mass a selection of that size can
    worst = D.rank_labels(-M, st.n_hi, st.n_lo)
    w = X.mass_stats(M, worst)
    assert w["recall"] < 1 and w["retained_mass"] < s["retained_mass"]
    # the draft's own selection lies between the two
    d = X.mass_stats(M, st.labels)
    assert w["retained_mass"] <= d["retained_mass"] <= s["retained_mass"] + 1e-15
    assert d["hi_mass"] + d["lo_mass"] == pytest.approx(d["retained_mass"], rel=1e-14)


def test_exact_attention_on_the_ideal_selection_beats_the_worst():
    # more true mass retained means a smaller sparsification error on the
    # same budget (not a theorem row by row; here the gap is wide)
    cfg = _cfg(gh=10, gw=9, hi=0.1, lo=0.2)
    q, k, v = _qkv(cfg, seed=6, scale=2.5)
    st = P.prepare_head(cfg, q, k, v)
    M = X.true_block_mass(st, q, k)
    best = X.error_split(st, q, k, v, labels=D.rank_labels(M, st.n_hi, st.n_lo))
    worst = X.error_split(st, q, k, v, labels=D.rank_labels(-M, st.n_hi, st.n_lo))
    assert best["sparsification"] < 0.5 * worst["sparsification"]


@pytest.mark.parametrize("shape", [(2, 16, 16, 4, 4), (21, 30, 52, 8, 16), (3, 5, 7, 4, 4), (2, 3, 5, 4, 8),
                                   (4, 9, 10, 4, 4), (2, 11, 13, 2, 8), (2, 30, 52, 16, 8), (1, 17, 33, 8, 16)])
@pytest.mark.parametrize("pack", [False, True])
def test_bench_token_blocks_match_the_oracle_geometry(shape, pack):
    import bench

    g = Geometry(*shape, pack_edges=pack)
    w = SimpleNamespace(frames=shape[0], grid_h=shape[1], grid_w=shape[2], win_h=shape[3], win_w=shape[4],
                        tokens=g.tokens)
    info = SimpleNamespace(n_wy=g.n_wy, n_wx=g.n_wx, n_full=g.n_full, flags=int(pack))
    got = bench.token_blocks(w, info, "cpu").numpy()
    idx = g.raster_index()
    want = np.empty(g.tokens, dtype=np.int64)
    for b in range(g.n_blocks):
        want[idx[b][idx[b] >= 0]] = b
    assert np.array_equal(got, want)


@pytest.mark.parametrize("pack,blocks", [(False, [1, 4, 7, 13, 22, 29]),     # of 30 windows (2 x 5 x 3)
                                         (True, [0, 5, 19, 20, 21, 22])])    # of 20 full + 3 stream blocks
def test_bench_fidelity_measure_matches_the_oracle(pack, blocks):
    # the benchmark's fp32 torch measurement, fed the oracle's labels, scores
    # and output, reproduces the oracle's float64 diagnostics on the same
    # sampled query blocks (ragged windows, two heads)
    import torch

    import bench

    cfg = _cfg(gh=10, gw=9, d=32, wh=2, ww=4, hi=0.1, lo=0.3)
    cfg.pack_edges = pack
    w = SimpleNamespace(batch=1, heads=2, tokens=cfg.frames * cfg.grid_h * cfg.grid_w, **vars(cfg))
    heads = [_qkv(cfg, seed=10 + h) for h in range(2)]
    sts = [P.prepare_head(cfg, *qkv) for qkv in heads]
    geo = sts[0].geo
    info = SimpleNamespace(n_blocks=geo.n_blocks, n_wy=geo.n_wy, n_wx=geo.n_wx, tau=sts[0].tau,
                           n_full=geo.n_full, flags=int(pack))
    assert geo.n_blocks == (23 if pack else 30)
    outs = [X.error_split(st, *qkv) for st, qkv in zip(sts, heads)]
    t = lambda i: torch.from_numpy(np.stack([qkv[i] for qkv in heads]))[None].float()
    method = torch.from_numpy(np.stack([o["method"] for o in outs]))[None].float()
    labels = torch.from_numpy(np.stack([st.labels for st in sts]))
    scores = torch.from_numpy(np.stack([st.scores for st in sts]))
    got = bench.fidelity(w, info, t(0), t(1), t(2), method, labels, scores, 0, blocks=blocks)

    rows = [np.concatenate([st.idx[i][st.valid[i]] for i in blocks]) for st in sts]
    num = lambda a, b: sum(float(((o[a][r] - o[b][r]) ** 2).sum()) for o, r in zip(outs, rows))
    den = sum(float((o["dense"][r] ** 2).sum()) for o, r in zip(outs, rows))
    assert got["sparsification_rel_l2"] == pytest.approx((num("sparse", "dense") / den) ** 0.5, rel=1e-4)
    assert got["quantization_rel_l2"] == pytest.approx((num("method", "sparse") / den) ** 0.5, rel=1e-3)
    assert got["total_rel_l2"] == pytest.approx((num("method", "dense") / den) ** 0.5, rel=1e-4)
    Ms = [X.true_block_mass(st, *qkv[:2])[blocks] for st, qkv in zip(sts, heads)]
    stats = [X.mass_stats(M, st.labels[blocks]) for M, st in zip(Ms, sts)]
    for key in ("hi_mass", "lo_mass", "retained_mass", "recall"):
        assert got[key] == pytest.approx(np.mean([s[key] for s in stats]), rel=1e-5), key
    cm = sum(float(((st.scores[blocks] - M) ** 2).sum()) for st, M in zip(sts, Ms))
    mm = sum(float((M ** 2).sum()) for M in Ms)
    assert got["draft_map_rel_fro"] == pytest.approx((cm / mm) ** 0.5, rel=1e-4)
    assert got["blocks_per_head"] == len(blocks) and got["rows_per_head"] == len(rows[0])


@pytest.mark.parametrize("pack", [False, True])
def test_bench_real_slot_flops_count_real_token_pairs(pack):
    # the benchmark's useful-work figure: for every retained (query block,
    # key block) pair, 4 d flops per pair of real tokens, counted here token
    # by token from the oracle geometry's raster indices (ragged windows)
    import torch

    import bench
    import block_sparse_mixed_amd as da2

    cfg = _cfg(frames=2, gh=10, gw=9, d=32, wh=2, ww=4)
    g = Geometry(cfg.frames, cfg.grid_h, cfg.grid_w, cfg.win_h, cfg.win_w, pack_edges=pack)
    w = SimpleNamespace(batch=1, heads=2, head_dim=cfg.head_dim, tokens=g.tokens, frames=cfg.frames,
                        grid_h=cfg.grid_h, grid_w=cfg.grid_w, win_h=cfg.win_h, win_w=cfg.win_w)
    info = SimpleNamespace(n_blocks=g.n_blocks, n_wy=g.n_wy, n_wx=g.n_wx, n_full=g.n_full, flags=int(pack))
    rng = np.random.default_rng(7)
    labels = rng.choice([da2.DA2_SKIP, da2.DA2_LO, da2.DA2_HI], size=(2, g.n_blocks, g.n_blocks))
    idx = g.raster_index()
    real = [int((idx[b] >= 0).sum()) for b in range(g.n_blocks)]
    want = {da2.DA2_HI: 0, da2.DA2_LO: 0}
    for h in range(2):
        for i in range(g.n_blocks):
            for j in range(g.n_blocks):
                if labels[h, i, j] in want:
                    want[labels[h, i, j]] += 4 * cfg.head_dim * real[i] * real[j]
    got = bench.real_slot_flops(w, info, torch.from_numpy(labels.astype(np.int8)))
    assert got == (want[da2.DA2_HI], want[da2.DA2_LO])
