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

import oracle_pool as OP
from gpu_cases import OUT_TOL, GpuRun, block_rows, check_prepare, compare_outputs, np64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def da2():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_sparse_mixed_amd as m
    return m


def _full_parity(da2, w, heads=None, att_blocks=None, run=None, states=None):
    run = GpuRun(da2, w) if run is None else run
    heads = range(run.bh) if heads is None else heads
    if states is None:
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
        assert len(same) >= 0.95 * run.nb, "too many label rows differ from the oracle's"
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


def _bits(t: torch.Tensor) -> np.ndarray:
    """bf16 CPU tensor -> its uint16 bit patterns."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _headline(da2, w, heads, blocks, inject_blocks):
    """The path the benchmark times, end to end: the GPU's own labels and its
    rank-ordered lists (no injection), then
      * codes, scales, pools, scores, labels and lists of `heads` against the oracle;
      * bf16 output of the same workspace = RNE of the fp32 output, every head;
      * fp32 output of `blocks` (None: all) of `heads` against the oracle,
        on every query block whose label row equals the oracle's (the others
        differ only inside the exemption band, checked above);
    and finally the oracle's labels injected, outputs on `inject_blocks`."""
    run = GpuRun(da2, w)
    out32 = run.attend(out_fp32=True)
    cfg_bf = da2.make_config(w.batch, w.heads, w.frames, w.grid_h, w.grid_w, w.head_dim, w.win_h, w.win_w,
                             w.budget_hi, w.budget_lo, out_dtype=da2.DA2_OUT_BF16)
    plan_bf = da2.da2_plan(cfg_bf)
    out16 = torch.empty(w.batch, w.heads, w.tokens, w.head_dim, dtype=torch.bfloat16, device="cuda")
    say(f"da2_attention bf16 {w.name}")
    da2.da2_attention(plan_bf, run.ws, out16)
    torch.cuda.synchronize()
    assert torch.equal(out16, out32.to(torch.bfloat16)), "bf16 output is not RNE of the fp32 output"
    lab = run.sec("labels", torch.int8, (run.bh, run.nb, run.nb))
    o = np64(out32.reshape(run.bh, w.tokens, w.head_dim))
    states = {}
    for bh in heads:
        st = run.oracle_head(bh)
        states[bh] = st
        say(f"check prepare {w.name} bh={bh}")
        check_prepare(run, bh, st)
        want_blocks = range(run.nb) if blocks is None else blocks
        same = (lab[bh] == st.labels).all(axis=1)
        use = [int(i) for i in want_blocks if same[i]]
        say(f"   {len(use)} of {len(want_blocks)} query blocks have the oracle's label row")
        assert len(use) >= 0.95 * len(want_blocks)
        b, h = divmod(bh, w.heads)
        rows, want = OP.attention_rows(w, _bits(run.qc[b, h]), _bits(run.kc[b, h]), _bits(run.vc[b, h]), use)
        say(f"   oracle rows {len(rows)} (pool of {OP.pool_size()})")
        assert np.array_equal(rows, np.sort(block_rows(st, use)))
        full = np.full((w.tokens, w.head_dim), np.nan)
        full[rows] = want
        worst, _ = compare_outputs(o[bh], full, rows)
        assert worst <= OUT_TOL, f"{w.name} bh={bh}: max |gpu - oracle| = {worst}"
    _full_parity(da2, w, heads=heads, att_blocks=inject_blocks, run=run, states=states)
    return run, states


@pytest.mark.timeout(900)
def test_wan_shape_end_to_end_all_blocks(da2):
    # every query block of two heads (incl. the partial edge windows and
    # frame boundaries), GPU labels and lists; then the injected-label path
    # on sampled blocks
    _headline(da2, S.WAN480, heads=[0, 7], blocks=None, inject_blocks=[0, 3, 15, 16, 170, 335])


@pytest.mark.timeout(900)
def test_hunyuan_shape_end_to_end_sampled(da2):
    # the largest shape: 24 heads x 118800 tokens, 990 blocks (the last row
    # of windows is 5 rows high); the first and last head, a seeded sample of
    # query blocks with at least 4096 real rows per head, incl. a partial
    # window (29) and the last block
    rng = np.random.default_rng(1)
    blocks = sorted(set(rng.choice(990, 36, replace=False).tolist()) | {0, 29, 500, 989})
    run, states = _headline(da2, S.HUNYUAN720, heads=[0, 23], blocks=blocks, inject_blocks=[0, 29, 500, 989])
    assert len(block_rows(states[0], blocks)) >= 4096


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
        # the other head sizes the plan accepts: 32 and 96 channels (one and
        # three MX groups of 32, the rest of the 128-channel tile zero)
        dataclasses.replace(S.TINY, name="d32", frames=2, grid_h=16, grid_w=32, win_h=8, win_w=16,
                            head_dim=32, budget_hi=0.25, budget_lo=0.25),
        dataclasses.replace(S.TINY, name="d96-ragged", frames=3, grid_h=13, grid_w=21, win_h=8, win_w=16,
                            head_dim=96, budget_hi=0.2, budget_lo=0.4),
        # windows of 64 and of 15 (odd) tokens: blocks of any size up to 128
        dataclasses.replace(S.TINY, name="win8x8", frames=2, grid_h=20, grid_w=20, win_h=8, win_w=8,
                            head_dim=128, budget_hi=0.15, budget_lo=0.35),
        dataclasses.replace(S.TINY, name="win3x5", frames=2, grid_h=10, grid_w=11, win_h=3, win_w=5,
                            head_dim=64, budget_hi=0.2, budget_lo=0.3),
    ]
    for w in cases:
        _full_parity(da2, w)


def test_set_labels_counts_rows_with_wrong_counts(da2):
    # the test hook rejects label rows whose hi/lo counts differ from the
    # plan's: status[0] is the number of such rows (reset on every call)
    w = S.TINY
    run = GpuRun(da2, w)
    st = run.oracle_head(0)
    bad = st.labels.copy()
    skip = np.flatnonzero(bad[3] == D.SKIP)[0]
    bad[3, skip] = D.HI                                  # one hi too many
    lo = np.flatnonzero(bad[5] == D.LO)[0]
    bad[5, lo] = D.SKIP                                  # one lo too few
    bad[9] = D.SKIP                                      # nothing retained
    assert run.set_labels(bad[None]) == 3
    assert run.set_labels(st.labels[None]) == 0
    out = np64(run.attend()[0, 0])
    worst, _ = compare_outputs(out, P.attention_raster(st), np.arange(w.tokens))
    assert worst <= OUT_TOL


def test_label_rows_with_too_few_labels_leave_valid_lists(da2):
    # the list sections filled with out-of-range block indices, then a label
    # row without any fp8 block: da2_set_labels reports it and fills that
    # row's fp8 list with block 0, so that every list entry names a real
    # block and the attention kernel reads only real tiles (that row's
    # outputs are unspecified); every other row still matches the oracle
    w = S.TINY
    run = GpuRun(da2, w)
    st = run.oracle_head(0)
    nb = run.nb
    for name, n in (("hi", st.n_hi), ("lo", st.n_lo)):
        da2.workspace_section(run.plan, run.ws, name, torch.int32, (run.bh, nb, n)).fill_(0x7FFFFFFF)
    bad = st.labels.copy()
    row = 5
    bad[row][bad[row] == D.HI] = D.SKIP
    assert run.set_labels(bad[None]) == 1
    hi = run.sec("hi", torch.int32, (run.bh, nb, st.n_hi))[0]
    lo = run.sec("lo", torch.int32, (run.bh, nb, st.n_lo))[0]
    assert (hi[row] == 0).all() and (hi >= 0).all() and (hi < nb).all() and (lo >= 0).all() and (lo < nb).all()
    out = np64(run.attend()[0, 0])
    good = [i for i in range(nb) if i != row]
    worst, _ = compare_outputs(out, P.attention_raster(st, blocks=good), block_rows(st, good))
    assert worst <= OUT_TOL


def test_nan_in_one_query_block_stays_in_that_block(da2):
    # a NaN in one query block's Q makes its draft scores NaN: its ranking
    # still labels n_hi + n_lo distinct real blocks (NaN scores sort below
    # every real one, so the order is by index), and every other query
    # block, which never reads that Q, matches the oracle on the inputs
    # without the NaN
    w = S.TINY
    q, k, v = S.make_qkv(w)
    qn = q.clone()
    g = lambda t: t.view(w.batch, w.heads, w.frames, w.grid_h, w.grid_w, w.head_dim)
    g(qn)[0, 0, 1, 5, 6, 7] = float("nan")               # frame 1, window (1, 1): block 21
    row = (1 * 4 + 1) * 4 + 1
    run = GpuRun(da2, w, qkv=(qn, k, v))
    st = P.prepare_head(w, np64(q[0, 0]), np64(k[0, 0]), np64(v[0, 0]))
    nb, n_hi, n_lo = run.nb, st.n_hi, st.n_lo
    C = run.sec("scores", torch.float64, (2, 1, nb, nb))[0, 0]
    assert np.isnan(C[row]).all() and np.isfinite(np.delete(C, row, axis=0)).all()
    lab = run.sec("labels", torch.int8, (1, nb, nb))[0]
    want_row = np.full(nb, D.SKIP, dtype=np.int8)
    want_row[:n_hi] = D.HI
    want_row[n_hi:n_hi + n_lo] = D.LO
    assert np.array_equal(lab[row], want_row)
    hi = run.sec("hi", torch.int32, (1, nb, n_hi))[0]
    lo = run.sec("lo", torch.int32, (1, nb, n_lo))[0]
    assert list(hi[row]) == list(range(n_hi)) and list(lo[row]) == list(range(n_hi, n_hi + n_lo))
    others = [i for i in range(nb) if i != row]
    same = [i for i in others if (lab[i] == st.labels[i]).all()]
    assert len(same) >= 0.95 * len(others)
    out = np64(run.attend()[0, 0])
    worst, _ = compare_outputs(out, P.attention_raster(st, blocks=same), block_rows(st, same))
    assert worst <= OUT_TOL


def test_zero_and_tiny_magnitude_blocks(da2):
    # windows of Q and K that are all zero, or scaled by 2^-70 so that the
    # fp8 score factor 2^(e_q + e_k) underflows fp32, next to ordinary ones;
    # partial windows give padded key slots (which must stay -inf). Ties in
    # the draft scores of the zero query block put the first key blocks,
    # including the tiny partial window 1, into its fp8 list.
    w = dataclasses.replace(S.TINY, name="zero-tiny", frames=3, grid_h=13, grid_w=21, win_h=8, win_w=16,
                            head_dim=128, budget_hi=0.2, budget_lo=0.4)
    q, k, v = S.make_qkv(w)
    grid = lambda t: t.view(w.batch, w.heads, w.frames, w.grid_h, w.grid_w, w.head_dim)
    tiny = 2.0 ** -70
    grid(q)[:, :, 0, 0:8, 0:16] = 0                      # block 0: zero queries
    grid(k)[:, :, 1, 8:13, 16:21] = 0                    # block 7: zero keys (partial window)
    grid(q)[:, :, 2, 0:8, 16:21] *= tiny                 # block 9: tiny queries (partial window)
    grid(k)[:, :, 0, 0:8, 16:21] *= tiny                 # block 1: tiny keys (partial window)
    grid(k)[:, :, 2, 8:13, 0:16] *= tiny                 # block 10: tiny keys
    run = GpuRun(da2, w, qkv=(q, k, v))
    st = run.oracle_head(0)
    assert st.ops["q8_exp"][0] == -127 and st.ops["q8_exp"][9] + st.ops["k8_exp"][1] < -140
    assert st.labels[0, 1] == D.HI and st.labels[9, 1] != D.SKIP
    assert np.ptp(st.scores[0]) == 0.0                   # the zero query block's scores all tie
    # these inputs' codes, pools, scores, labels and lists, then attention
    # with the GPU's own labels, then with the oracle's injected
    check_prepare(run, 0, st)
    out = run.attend()
    assert torch.isfinite(out).all()
    lab = run.sec("labels", torch.int8, (1, run.nb, run.nb))[0]
    same = np.flatnonzero((lab == st.labels).all(axis=1))
    worst, _ = compare_outputs(np64(out[0, 0]), P.attention_raster(st, blocks=same), block_rows(st, same))
    assert worst <= OUT_TOL
    _full_parity(da2, w, run=run, states={0: st})


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


@pytest.mark.parametrize("grid", [40, 60, 66])
def test_ranking_ties_at_every_sort_size(da2, grid):
    # 2x2-token windows give 400, 900 and 1089 blocks: the one-wave ranking
    # with 8 and 16 pairs a lane and the workgroup ranking. Copies of one key
    # window have equal logits in both maps, so they tie in every row, in
    # the fp8 list, in the MXFP4 list and across both budget thresholds;
    # the rows of all-zero query windows are ties throughout. The order of
    # equal scores, by index, then decides labels and lists.
    w = dataclasses.replace(S.TINY, name=f"ties{grid}", frames=1, grid_h=grid, grid_w=grid, win_h=2, win_w=2,
                            head_dim=64, budget_hi=0.1, budget_lo=0.2)
    q, k, v = S.make_qkv(w)
    g = lambda t: t.view(w.batch, w.heads, w.grid_h, w.grid_w, w.head_dim)
    src = g(k)[:, :, 2:4, 4:6].clone()
    copies = []
    for y in range(0, grid, 6):
        x = (3 * y) % grid
        g(k)[:, :, y:y + 2, x:x + 2] = src                            # copies of key window (1, 2)
        copies.append((y // 2) * (grid // 2) + x // 2)
    g(q)[:, :, 0:2, 0:2] = 0                                          # zero query windows
    g(q)[:, :, grid - 2:grid, 10:12] = 0
    run = GpuRun(da2, w, qkv=(q, k, v))
    say(f"check prepare {w.name} nb={run.nb}")
    st = run.oracle_head(0)
    nb, n_hi, n_ret = run.nb, st.n_hi, st.n_hi + st.n_lo
    rank = np.argsort(np.lexsort((np.broadcast_to(np.arange(nb), st.scores.shape), -st.scores), axis=-1), axis=-1)
    rc = rank[:, copies]
    assert np.ptp(st.scores[0]) == 0.0 and np.ptp(st.scores[1, copies]) == 0.0
    for t in (n_hi, n_ret):                                           # ties across each threshold
        assert ((rc.min(1) < t) & (rc.max(1) >= t)).sum() > 0
    check_prepare(run, 0, st)


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
