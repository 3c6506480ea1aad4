"""Pins for oracle.geometry / oracle.draft: bijection, torch pooling, closed forms,
rigged rankings, brute-force sort."""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as TF

from oracle import draft as D
from oracle.geometry import Geometry, gather_blocks


@pytest.mark.parametrize("shape,expect", [
    ((2, 16, 16, 4, 4), (32, 16, 512, 512)),           # Tiny
    ((5, 32, 32, 8, 16), (40, 128, 5120, 5120)),        # Small
    ((21, 30, 52, 8, 16), (336, 128, 43008, 32760)),    # Wan-480p shape
    ((33, 45, 80, 8, 16), (990, 128, 126720, 118800)),  # Hunyuan-720p shape
])
def test_geometry_counts_and_bijection(shape, expect):
    g = Geometry(*shape)
    idx = g.raster_index()
    assert (g.n_blocks, g.block_size, idx.size, g.tokens) == expect
    real = idx[idx >= 0]
    assert real.size == g.tokens
    assert np.array_equal(np.sort(real), np.arange(g.tokens))


def test_geometry_landmarks_wan():
    g = Geometry(21, 30, 52, 8, 16)
    idx = g.raster_index()
    assert idx[0, 0] == 0 and idx[0, 1] == 1 and idx[0, 16] == 52      # slot 16 = next row
    assert idx[1, 0] == 16                                              # second window starts at x=16
    corner = (0 * 4 + 3) * 4 + 3                                        # frame 0, last window row/col
    assert (idx[corner] >= 0).sum() == 6 * 4                            # rows 24..29, cols 48..51
    assert idx[4 * 4, 0] == 30 * 52                                     # first window of frame 1


@pytest.mark.parametrize("shape,expect", [
    ((2, 16, 16, 4, 4), (32, 32)),          # Tiny: divisible, no edge stream
    ((5, 32, 32, 8, 16), (40, 40)),         # Small: divisible
    ((21, 30, 52, 8, 16), (256, 189)),      # Wan-480p shape: 9 full windows a frame + 67 stream blocks
    ((33, 45, 80, 8, 16), (929, 825)),      # Hunyuan-720p shape: 25 a frame + 104
    ((3, 5, 7, 4, 4), (7, 3)),              # ragged both ways, small
    ((2, 3, 5, 4, 8), (1, 0)),              # grid smaller than a window: stream only
])
def test_packed_geometry_counts_and_bijection(shape, expect):
    g = Geometry(*shape, pack_edges=True)
    idx = g.raster_index()
    assert (g.n_blocks, g.n_full) == expect
    assert g.n_blocks == -(-g.tokens // g.block_size)          # no block wasted
    real = idx[idx >= 0]
    assert np.array_equal(np.sort(real), np.arange(g.tokens))
    valid = idx >= 0
    assert valid[:-1].all()                                     # only the last block may be short
    assert valid[-1].sum() == g.tokens - (g.n_blocks - 1) * g.block_size
    # the full windows are the padded geometry's full windows, in order
    p = Geometry(*shape)
    pidx = p.raster_index()
    full = pidx[(pidx >= 0).all(axis=1)]
    assert np.array_equal(idx[:g.n_full], full)
    if shape[1] % shape[3] == 0 and shape[2] % shape[4] == 0:
        assert np.array_equal(idx, pidx)


def test_packed_geometry_landmarks_wan():
    g = Geometry(21, 30, 52, 8, 16, pack_edges=True)
    idx = g.raster_index()
    assert idx[0, 0] == 0 and idx[1, 0] == 16 and idx[3, 0] == 8 * 52   # full windows (0,0) (0,1) (1,0)
    assert idx[9, 0] == 30 * 52                                          # frame 1's first full window
    e = idx[189]                                                         # first block of the edge stream:
    assert e[0] == 48 and e[3] == 51 and e[4] == 52 + 48                 # window (0,3), 8 x 4 tokens
    assert e[32] == 8 * 52 + 48 and e[64] == 16 * 52 + 48                # windows (1,3), (2,3)
    assert e[96] == 24 * 52 and e[112] == 25 * 52                        # window (3,0): 6 x 16 tokens
    assert idx[255, 119] == 32759 and (idx[255, 120:] == -1).all()       # frame 20's last corner token


def _pool_torch(frame, ph, pw):
    """frame [H, W, d] -> avg/max over (ph, pw) windows with partial edge windows (ceil)."""
    x = torch.from_numpy(frame).permute(2, 0, 1)[None]
    avg = TF.avg_pool2d(x, (ph, pw), stride=(ph, pw), ceil_mode=True)
    mx = TF.max_pool2d(x, (ph, pw), stride=(ph, pw), ceil_mode=True)
    return avg[0].permute(1, 2, 0).numpy(), mx[0].permute(1, 2, 0).numpy()


@pytest.mark.parametrize("hw,win", [((16, 16), (4, 4)), ((30, 52), (8, 16)), ((45, 80), (8, 16))])
def test_pool_matches_torch_pooling(hw, win):
    rng = np.random.default_rng(2)
    T, d = 2, 8
    H, W = hw
    g = Geometry(T, H, W, *win)
    x = rng.normal(size=(T * H * W, d))
    idx = g.raster_index()
    mean, mx = D.pool_blocks(gather_blocks(x, idx), idx >= 0)
    for t in range(T):
        a, m = _pool_torch(x[t * H * W:(t + 1) * H * W].reshape(H, W, d), *win)
        sl = slice(t * g.n_wy * g.n_wx, (t + 1) * g.n_wy * g.n_wx)
        np.testing.assert_allclose(mean[sl], a.reshape(-1, d), rtol=1e-13, atol=1e-13)
        np.testing.assert_array_equal(mx[sl], m.reshape(-1, d))


def test_pool_closed_forms():
    g = Geometry(1, 8, 16, 8, 16)
    yy, xx = np.meshgrid(np.arange(8), np.arange(16), indexing="ij")
    affine = (3.0 * yy + 0.5 * xx - 2.0).reshape(-1, 1)
    const = np.full((128, 1), 1.75)
    x = np.concatenate([affine, const], axis=1)
    idx = g.raster_index()
    mean, mx = D.pool_blocks(gather_blocks(x, idx), idx >= 0)
    assert mean[0, 0] == pytest.approx(3.0 * 3.5 + 0.5 * 7.5 - 2.0, abs=1e-12)   # value at centre
    assert mx[0, 0] == 3.0 * 7 + 0.5 * 15 - 2.0
    assert mean[0, 1] == 1.75 and mx[0, 1] == 1.75


def test_draft_scores_closed_form_two_blocks():
    tau = 0.7
    qa = np.array([[1.0, 0.0]])
    ka = np.array([[1.0, 0.0], [0.0, 0.0]])
    qm = np.array([[0.0, 2.0]])
    km = np.array([[0.0, 0.0], [0.0, 1.0]])
    C = D.draft_scores(np.repeat(qa, 2, 0), np.repeat(qm, 2, 0), ka, km, tau)
    a_avg = [math.exp(tau) / (math.exp(tau) + 1), 1 / (math.exp(tau) + 1)]
    a_max = [1 / (1 + math.exp(2 * tau)), math.exp(2 * tau) / (1 + math.exp(2 * tau))]
    expect = [0.5 * (a_avg[0] + a_max[0]), 0.5 * (a_avg[1] + a_max[1])]
    np.testing.assert_allclose(C[0], expect, rtol=1e-14)


def test_draft_rows_stochastic_and_uniform_for_identical_keys():
    rng = np.random.default_rng(3)
    qa, qm = rng.normal(size=(6, 8)), rng.normal(size=(6, 8))
    ka, km = rng.normal(size=(6, 8)), rng.normal(size=(6, 8))
    C = D.draft_scores(qa, qm, ka, km, 0.3)
    np.testing.assert_allclose(C.sum(1), 1.0, rtol=1e-14)
    same = np.tile(rng.normal(size=(1, 8)), (6, 1))
    C2 = D.draft_scores(qa, qm, same, same, 0.3)
    np.testing.assert_allclose(C2, 1.0 / 6, rtol=1e-14)


def test_draft_direction_and_both_maps_count():
    # query block i points at key block perm[i] (not a symmetric permutation):
    # a transposed product would pick perm^-1(i) instead
    perm = np.array([1, 2, 3, 4, 0])
    eye = np.eye(5) * 10
    zeros = np.zeros((5, 5))
    for which in ("avg", "max", "both"):
        qa = eye[perm] if which in ("avg", "both") else zeros
        qm = eye[perm] if which in ("max", "both") else zeros
        C = D.draft_scores(qa, qm, eye, eye, 1.0)
        assert np.array_equal(C.argmax(1), perm), which


def test_budget_counts_closed_forms():
    assert D.budget_counts(32, 0.25, 0.25) == (8, 8)
    assert D.budget_counts(40, 0.10, 0.30) == (4, 12)
    assert D.budget_counts(336, 0.15, 0.35) == (50, 118)
    assert D.budget_counts(990, 0.10, 0.20) == (99, 198)
    sweep = {(0.05, 0.0): (17, 0), (0.05, 0.2): (17, 67), (0.05, 0.4): (17, 134),
             (0.10, 0.0): (34, 0), (0.10, 0.2): (34, 67), (0.10, 0.4): (34, 134),
             (0.25, 0.0): (84, 0), (0.25, 0.2): (84, 67), (0.25, 0.4): (84, 134),
             (1.0, 0.0): (336, 0), (1.0, 0.2): (336, 0), (1.0, 0.4): (336, 0), (0.0, 1.0): (0, 336)}
    for (h, l), want in sweep.items():
        assert D.budget_counts(336, h, l) == want, (h, l)
    with pytest.raises(ValueError):
        D.budget_counts(336, 0.0, 0.001)


def test_rank_brute_force_with_ties():
    rng = np.random.default_rng(4)
    nb = 23
    C = rng.integers(0, 6, size=(nb, nb)).astype(float) / 5.0      # many exact ties
    n_hi, n_lo = 5, 7
    lab = D.rank_labels(C, n_hi, n_lo)
    for i in range(nb):
        order = sorted(range(nb), key=lambda j: (-C[i, j], j))
        want = np.zeros(nb, dtype=np.int8)
        for r, j in enumerate(order):
            want[j] = D.HI if r < n_hi else (D.LO if r < n_hi + n_lo else D.SKIP)
        assert np.array_equal(lab[i], want)
    assert np.all((lab == D.HI).sum(1) == n_hi) and np.all((lab == D.LO).sum(1) == n_lo)


def test_rank_orders_scores_and_budget_extremes():
    rng = np.random.default_rng(5)
    C = rng.random((30, 30))
    lab = D.rank_labels(C, 6, 9)
    for i in range(30):
        assert C[i, lab[i] == D.HI].min() >= C[i, lab[i] == D.LO].max() >= C[i, lab[i] == D.SKIP].max()
    assert np.all(D.rank_labels(C, *D.budget_counts(30, 1.0, 0.0)) == D.HI)
    assert np.all(D.rank_labels(C, *D.budget_counts(30, 0.3, 0.7)) != D.SKIP)


def test_exemption_band():
    C = np.array([[0.4, 0.3, 0.2, 0.1 + 1e-7, 0.1]])
    ex = D.exemption_mask(C, 3, 0)           # threshold between ranks 3 and 4: 0.2 vs 0.1+1e-7
    assert not ex.any()
    ex = D.exemption_mask(C, 4, 0)           # between 0.1+1e-7 and 0.1: both within 1e-5 relative
    assert ex[0].tolist() == [False, False, False, True, True]
