"""GPU parity through the C ABI against the CPU oracle (MI355X only).

Bars: quantized codes, scales and (outside the 1e-5 exemption band) labels
bit-exact; pooled values and block scores to float64 rounding; outputs within
2e-3 max-abs of the oracle on the same quantized operands, with the oracle's
labels injected and end to end.
"""

import dataclasses

import numpy as np
import pytest
import torch

import synthetic as S
from oracle import draft as D
from oracle import pipeline as P

from gpu_cases import OUT_TOL, GpuRun, block_rows, check_prepare, compare_outputs, np64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def da2():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_sparse_mixed_amd as m
    return m


def _full_parity(da2, w, heads=None, att_blocks=None):
    run = GpuRun(da2, w)
    heads = range(run.bh) if heads is None else heads
    states = {bh: run.oracle_head(bh) for bh in heads}
    for bh, st in states.items():
        say(f"check prepare {w.name} bh={bh}")
        check_prepare(run, bh, st)
    # attention with the oracle's own labels injected
    labels = np.zeros((run.bh, run.nb, run.nb), dtype=np.int8)
    full_labels = {bh: st.labels for bh, st in states.items()}
    gpu_lab = run.sec("labels", torch.int8, (run.bh, run.nb, run.nb))
    for bh in range(run.bh):
        labels[bh] = full_labels.get(bh, gpu_lab[bh])
    assert run.set_labels(labels) == 0
    out = np64(run.attend().reshape(run.bh, w.tokens, w.head_dim))
    for bh, st in states.items():
        blocks = range(run.nb) if att_blocks is None else att_blocks
        want = P.attention_raster(st, blocks=blocks)
        rows = block_rows(st, blocks)
        worst, nbad = compare_outputs(out[bh], want, rows)
        assert worst <= OUT_TOL, f"{w.name} bh={bh}: max |gpu - oracle| = {worst}"
    return run, states, out


def test_tiny_full(da2):
    _full_parity(da2, S.TINY)


def test_small_full(da2):
    _full_parity(da2, S.SMALL)


def test_end_to_end_small_and_determinism(da2):
    w = S.SMALL
    run = GpuRun(da2, w)
    out1 = run.attend()
    out2 = run.attend()
    assert torch.equal(out1, out2), "two launches differ"
    lab = run.sec("labels", torch.int8, (run.bh, run.nb, run.nb))
    o = np64(out1.reshape(run.bh, w.tokens, w.head_dim))
    for bh in range(run.bh):
        st = run.oracle_head(bh)
        same = np.flatnonzero((lab[bh] == st.labels).all(axis=1))
        want = P.attention_raster(st, blocks=same)
        worst, _ = compare_outputs(o[bh], want, block_rows(st, same))
        assert worst <= OUT_TOL


def test_bf16_output_is_rne_of_fp32(da2):
    w = S.SMALL
    run = GpuRun(da2, w)
    o32 = run.attend(out_fp32=True)
    cfg_bf = da2.make_config(w.batch, w.heads, w.frames, w.grid_h, w.grid_w, w.head_dim, w.win_h, w.win_w,
                             w.budget_hi, w.budget_lo, out_dtype=da2.DA2_OUT_BF16)
    plan_bf = da2.da2_plan(cfg_bf)
    o16 = torch.empty(w.batch, w.heads, w.tokens, w.head_dim, dtype=torch.bfloat16, device="cuda")
    say("da2_attention bf16 small")
    da2.da2_attention(plan_bf, run.ws, o16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16))


def test_wan_shape_sampled(da2):
    # full-size launch; codes/labels for two heads, outputs on sampled query
    # blocks including the partial edge windows (3, 15) and a frame boundary
    _full_parity(da2, S.WAN480, heads=[0, 7], att_blocks=[0, 3, 15, 16, 170, 335])


def test_hunyuan_shape_sampled(da2):
    # the largest shape: 24 heads x 118800 tokens, 990 blocks (rows of windows
    # partial in y); codes/labels for the first and last head, outputs on
    # sampled query blocks including a partial window (29) and the last block
    _full_parity(da2, S.HUNYUAN720, heads=[0, 23], att_blocks=[0, 29, 500, 989])


@pytest.mark.parametrize("hi,lo", [(0.05, 0.0), (0.05, 0.4), (0.1, 0.2), (0.25, 0.2), (0.25, 0.4), (1.0, 0.0),
                                   (0.0, 1.0)])
def test_wan_sweep_points_sampled(da2, hi, lo):
    w = S.with_budgets(S.WAN480, hi, lo)
    _full_parity(da2, w, heads=[3], att_blocks=[0, 15, 200])


def test_edge_shapes(da2):
    # one frame smaller than a window; odd sizes; head_dim 64 with 128-token windows
    cases = [
        dataclasses.replace(S.TINY, name="subwindow", frames=1, grid_h=5, grid_w=7, win_h=8, win_w=16,
                            budget_hi=1.0, budget_lo=0.0),
        dataclasses.replace(S.TINY, name="ragged", frames=3, grid_h=13, grid_w=21, win_h=8, win_w=16,
                            head_dim=128, budget_hi=0.2, budget_lo=0.4),
        dataclasses.replace(S.TINY, name="d64w128", frames=2, grid_h=16, grid_w=32, win_h=8, win_w=16,
                            head_dim=64, budget_hi=0.25, budget_lo=0.5),
        dataclasses.replace(S.TINY, name="batch2", batch=2, heads=3, frames=2, grid_h=8, grid_w=8),
    ]
    for w in cases:
        _full_parity(da2, w)


@pytest.mark.parametrize("grid", [66, 94])
def test_prepare_large_block_counts(da2, grid):
    # 2x2-token windows give 1089 and 2209 blocks: the ranking sorts 2048 and
    # 4096 (score, index) pairs per row (eight and sixteen per thread), past
    # the sizes the video workloads reach
    w = dataclasses.replace(S.TINY, name=f"blocks{grid}", frames=1, grid_h=grid, grid_w=grid, win_h=2, win_w=2,
                            head_dim=64, budget_hi=0.1, budget_lo=0.2)
    run = GpuRun(da2, w)
    say(f"check prepare {w.name} nb={run.nb}")
    check_prepare(run, 0, run.oracle_head(0))


def test_attention_long_tile_lists(da2):
    # 1089 blocks of 4 tokens, 327 retained per query block (109 fp8, 218
    # MXFP4): long tile lists whose tiles are 124/128 padding, end to end on
    # sampled query blocks
    w = dataclasses.replace(S.TINY, name="blocks66", frames=1, grid_h=66, grid_w=66, win_h=2, win_w=2,
                            head_dim=64, budget_hi=0.1, budget_lo=0.2)
    _full_parity(da2, w, heads=[0], att_blocks=[0, 17, 544, 1088])


def test_packed_edges_full(da2):
    # packed edge windows: stream blocks mixing windows and frames, a short
    # last block; 128-token windows with d = 128, and 16-token windows
    cases = [
        dataclasses.replace(S.WAN480, name="packed-3f", heads=2, frames=3, pack_edges=True),
        dataclasses.replace(S.TINY, name="packed-small-win", frames=2, grid_h=10, grid_w=9, win_h=4, win_w=4,
                            budget_hi=0.25, budget_lo=0.25, pack_edges=True),
        dataclasses.replace(S.TINY, name="packed-subwindow", frames=2, grid_h=5, grid_w=7, win_h=8, win_w=16,
                            budget_hi=1.0, budget_lo=0.0, pack_edges=True),
    ]
    for w in cases:
        _full_parity(da2, w)


def test_wan_shape_packed_sampled(da2):
    # full-size packed launch: 189 full windows + 67 stream blocks (the last
    # one 120 tokens); outputs on full-window, stream and last blocks
    w = dataclasses.replace(S.WAN480, name="wan480p-packed", pack_edges=True)
    _full_parity(da2, w, heads=[0, 11], att_blocks=[0, 188, 189, 200, 255])


def test_graph_capture_replays_match_eager(da2):
    # the whole step (prepare + attention) captured in a HIP graph: every
    # replay, with other eager work and synchronisations between them and
    # new input values copied into the captured buffers, matches an eager
    # call on the same values bit for bit (the library enqueues kernels only)
    w = S.SMALL
    run = GpuRun(da2, w)
    q2, k2, v2 = (t.cuda() for t in S.make_qkv(dataclasses.replace(w, seed=5)))
    inputs = [(run.q.clone(), run.k.clone(), run.v.clone()), (q2, k2, v2)]
    out = torch.empty(w.batch, w.heads, w.tokens, w.head_dim, dtype=torch.float32, device="cuda")
    want = []
    for q, k, v in inputs:
        da2.da2_prepare(run.plan, q, k, v, run.ws)
        da2.da2_attention(run.plan, run.ws, out)
        torch.cuda.synchronize()
        want.append(out.clone())
    assert not torch.equal(want[0], want[1])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on a side stream before capture
        da2.da2_prepare(run.plan, run.q, run.k, run.v, run.ws)
        da2.da2_attention(run.plan, run.ws, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say("capture prepare + attention (small)")
    with torch.cuda.graph(graph):
        da2.da2_prepare(run.plan, run.q, run.k, run.v, run.ws)
        da2.da2_attention(run.plan, run.ws, out)
    torch.cuda.synchronize()
    for rep in range(4):
        i = rep % 2
        for dst, src in zip((run.q, run.k, run.v), inputs[i]):
            dst.copy_(src)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"replay {rep} (inputs {i})")
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want[i]), f"replay {rep} differs from the eager result"


def test_strided_inputs_match_contiguous(da2):
    # q, k, v as [B, N, H, d] storage viewed as [B, H, N, d], and as slices
    # of one fused [B, N, 3, H, d] tensor: the same values give the same
    # output, bit for bit, as the contiguous layout (batch 2, packed and not)
    w = dataclasses.replace(S.SMALL, name="strided", batch=2)
    q, k, v = (t.cuda() for t in S.make_qkv(w))
    args = (w.frames, w.grid_h, w.grid_w, w.win_h, w.win_w, w.budget_hi, w.budget_lo)
    for flags in (0, da2.DA2_FLAG_PACK_EDGES):
        say(f"contiguous, flags={flags}")
        ref = da2.attention(q, k, v, *args, out_dtype=torch.float32, flags=flags)
        bnhd = [t.transpose(1, 2).contiguous().transpose(1, 2) for t in (q, k, v)]
        fused = torch.stack([t.transpose(1, 2) for t in (q, k, v)], dim=2).contiguous()   # [B, N, 3, H, d]
        views = [fused[:, :, i].transpose(1, 2) for i in range(3)]
        for name, (qq, kk, vv) in (("bnhd", bnhd), ("fused-qkv", views)):
            assert not qq.is_contiguous() and torch.equal(qq, q)
            say(f"{name} strides {tuple(qq.stride())}, flags={flags}")
            out = da2.attention(qq, kk, vv, *args, out_dtype=torch.float32, flags=flags)
            assert out.stride() == qq.stride()
            torch.cuda.synchronize()
            assert torch.equal(out, ref), f"{name}: output differs from the contiguous layout"
