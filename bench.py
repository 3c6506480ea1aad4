"""Benchmark of the DraftAttention2 hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
da2_prepare (fused operand preparation + draft map + shared ranking) and
da2_attention (phased block-sparse attention), on the Wan-480p-shaped
workload (12 heads, 21 x 30 x 52 latent tokens, d = 128, 8x16 windows,
budgets 15 % fp8 / 35 % MXFP4 / 50 % skip). Inputs are resident in HBM
before the timed region.

Prints one JSON line. `value` is the dense-equivalent attention throughput of
the whole step, 4*B*H*N^2*d / step time. The `roofline` object is for the
attention kernel (the dominant one): executed (algorithmic) MFMA flops per
launch over its average launch time, against the blended fp8/MXFP4 peak of
the step's hi/lo mix, T* = F_hi / P_fp8 + F_lo / P_fp4.

The `traffic` field is the attention kernel's HBM bytes per launch from the
FETCH_SIZE and WRITE_SIZE counters (rocprofv3 --pmc), each scaled by what the
same counter reads for a plain streaming kernel of known size
(`--copy-calibration`). Those figures are kept in
profiles/attn_wan480p_traffic.md together with the SHA-256 of the attention
kernel's sources (attn.hip, common.hpp) they were taken on; when the source has changed since, the
field is null.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload wan480p]
       [--no-cpu-baseline] [--cpu-heads H] [--cpu-workers P]
       python bench.py --copy-calibration   (counter calibration run only)
       python bench.py --all-configs        (every workload at its own budgets, one JSON
                                             line each, with the error against dense fp32)
       python bench.py --dit-block          (the DiT attention sublayer: fused custom op,
                                             unfused layout copies, dense SDPA)
       python bench.py --sweep              (budget sweep on the Wan-480p shape, one
                                             JSON line per point, with the error
                                             against dense fp32 attention)
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)

P_FP8 = 5.0e15       # MI355X dense fp8 MFMA, FLOP/s (published)
P_FP4 = 10.1e15      # MI355X dense fp4 MFMA, FLOP/s (published)
P_BF16 = 2.5e15      # MI355X dense bf16 MFMA, FLOP/s (published)
METRIC = "dense-equiv attention TFLOPS + % blended MFMA roofline (Wan-480p shape)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan480p")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=1,
                    help="heads of the workload the CPU oracle baseline runs in full (preparation and every query block)")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="oracle processes (0: the CPUs this process may use, at most 16)")
    ap.add_argument("--error-rows", type=int, default=2048,
                    help="query rows per head sampled for the error against dense fp32 attention")
    ap.add_argument("--all-configs", action="store_true",
                    help="one JSON line per workload (tiny, small, wan480p, hunyuan720p): times and error vs dense fp32")
    ap.add_argument("--dit-block", action="store_true",
                    help="time the attention sublayer of a DiT block at the workload's shape (QKV projection, "
                         "attention, output projection; random weights): the fused custom op, the unfused "
                         "sequence with layout copies, and dense torch SDPA")
    ap.add_argument("--sweep", action="store_true",
                    help="budget sweep on the Wan-480p shape: time and error vs dense fp32 per point")
    ap.add_argument("--sweep-rows", type=int, default=2048,
                    help="query rows per head sampled for the error against dense attention")
    ap.add_argument("--sweep-blocks", type=int, default=16,
                    help="whole query blocks per head sampled for the error split and draft fidelity")
    ap.add_argument("--pack-edges", action="store_true",
                    help="packed edge windows (partial windows streamed into shared blocks) for the timed line and the sweep")
    ap.add_argument("--no-alt-layout", action="store_true",
                    help="do not also time the other block layout")
    ap.add_argument("--budgets", type=float, nargs=2, metavar=("HI", "LO"),
                    help="override the workload's hi and lo budgets (fractions of key blocks) for the timed line; "
                         "the workload is then named with them, and its traffic figure is not reported")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a streaming kernel of known size (read 1 GiB, write 1 GiB), for counter scaling")
    return ap.parse_args()


# the attention kernel's sources: the kernel file and the geometry helpers it includes
ATTN_SOURCES = [os.path.join(HERE, "block_sparse_mixed_amd", "csrc", f) for f in ("attn.hip", "common.hpp")]
TRAFFIC_FILE = os.path.join(HERE, "profiles", "attn_wan480p_traffic.md")


def attn_source_sha256():
    """SHA-256 of the attention kernel's sources, concatenated in order."""
    h = hashlib.sha256()
    for path in ATTN_SOURCES:
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(workload):
    """Scaled HBM bytes per attention launch from the committed counter summary,
    or None when it is missing, for another workload, or for other kernel source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            text = fh.read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ":" in line:
            key, val = line[2:].split(":", 1)
            fields[key.strip()] = val.strip().strip("`")
    if fields.get("workload") != workload or fields.get("attn_source_sha256") != attn_source_sha256():
        return None
    try:
        return float(fields["scaled_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration():
    import torch
    n = 1 << 28                     # 2^28 fp32 = 1 GiB read + 1 GiB written per launch
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"kernel": "torch.mul(src, 1.0, out=dst)", "read_bytes": 4 * n,
                                           "write_bytes": 4 * n, "launches": 3}}), flush=True)


def flops(w, nb, n_hi, n_lo):
    B, H, N, d = w.batch, w.heads, w.tokens, w.head_dim
    dense = 4.0 * B * H * N * N * d
    tile = 128.0
    f_hi = 4.0 * B * H * nb * n_hi * tile * tile * d
    f_lo = 4.0 * B * H * nb * n_lo * tile * tile * d
    return dense, f_hi, f_lo


def real_slot_flops(w, info, labels):
    """MFMA work on real key and query slots only, (F_hi, F_lo): per retained
    (query block, key block) pair 4 d n_q n_k flops with the blocks' real
    token counts, where the executed figures count all 128 x 128 slots."""
    import torch

    import block_sparse_mixed_amd as da2
    cnt = torch.bincount(token_blocks(w, info, "cpu"), minlength=info.n_blocks).double()
    out = []
    for lab in (da2.DA2_HI, da2.DA2_LO):
        m = (labels == lab).double()
        out.append(4.0 * w.head_dim * float(torch.einsum("i,bij,j->", cnt, m, cnt)))
    return tuple(out)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_worker_init():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)
    import oracle.pipeline  # noqa: F401  (imported before the timed region)


_ORACLE_HEADS = {}


def _oracle_ready(_):
    time.sleep(0.1)         # long enough that every worker takes one of these
    return os.getpid()


def _oracle_chunk(task):
    """One worker's share of the oracle baseline: the whole preparation of
    the head (once per worker and head), then attention for its query blocks.
    Returns (head, preparation seconds or 0 when cached, attention seconds,
    worker pid)."""
    import numpy as np

    from oracle import pipeline as P
    cfg, head, bits, blocks = task
    prep = 0.0
    if head not in _ORACLE_HEADS:
        t0 = time.perf_counter()
        f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        import types
        _ORACLE_HEADS[head] = P.prepare_head(types.SimpleNamespace(**cfg), *(f(b) for b in bits))
        prep = time.perf_counter() - t0
    t0 = time.perf_counter()
    P.attention_raster(_ORACLE_HEADS[head], blocks=blocks)
    return head, prep, time.perf_counter() - t0, os.getpid()


def cpu_baseline(w, q, k, v, heads, workers):
    """The oracle as it stands, timed on the host CPUs: a pool of `workers`
    spawned processes with one BLAS thread each runs the whole path
    (geometry, pooling, draft map, ranking, quantization, attention) for
    every query block of the first `heads` heads. Each worker prepares the
    heads it serves itself (in parallel with the others), then attends its
    share of the query blocks. The value is the dense-equivalent work of
    those heads over the measured wall time (heads carry equal work, so it
    is the rate of the whole workload)."""
    import concurrent.futures as cf
    import multiprocessing as mp

    import numpy as np

    from oracle.geometry import Geometry
    cfg = {k2: getattr(w, k2) for k2 in ("frames", "grid_h", "grid_w", "head_dim", "win_h", "win_w",
                                          "budget_hi", "budget_lo", "pack_edges")}
    nb = Geometry(w.frames, w.grid_h, w.grid_w, w.win_h, w.win_w, pack_edges=w.pack_edges).n_blocks
    bits = lambda t, h: t[0, h].contiguous().view(torch_int16()).numpy().view(np.uint16)
    per_head = max(1, workers // heads)
    tasks = []
    for h in range(heads):
        b3 = (bits(q, h), bits(k, h), bits(v, h))
        for c in range(per_head):
            tasks.append((cfg, h, b3, list(range(c, nb, per_head))))
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(max_workers=workers, mp_context=ctx, initializer=_oracle_worker_init) as ex:
        list(ex.map(_oracle_ready, range(2 * workers)))             # every worker up, imports done
        t0 = time.perf_counter()
        res = list(ex.map(_oracle_chunk, tasks))
        wall = time.perf_counter() - t0
    preps = [r[1] for r in res if r[1] > 0]
    atts = [r[2] for r in res]
    dense, _, _ = flops(w, nb, 0, 0)
    dense_heads = dense * heads / (w.batch * w.heads)
    return {
        "value": dense_heads / wall / 1e12,
        "unit": "TFLOP/s",
        "cores": len({r[3] for r in res}),
        "kind": "oracle",
        "sample": (f"{heads} of {w.batch * w.heads} heads in full (preparation + all {nb} query blocks), "
                   f"{workers} spawned processes with 1 BLAS thread each; wall {wall:.1f} s"),
        "cpu_model": _cpu_model(),
        "wall_s": wall,
        # per stage: one whole-head preparation (each worker prepares the heads
        # it serves, all at once), and attention in core-seconds per query block
        "stage_s": {"prepare_per_head": sum(preps) / max(1, len(preps)),
                    "attention_core_s_per_block": sum(atts) / (heads * nb)},
        "extrapolated_step_s": wall * (w.batch * w.heads) / heads,
    }


def torch_int16():
    import torch
    return torch.int16


def dense_error(q, k, v, out, tau, rows_per_head, seed=0):
    """Error of `out` against dense fp32 softmax attention over the same bf16
    inputs, on a seeded sample of query rows of every head: max-abs,
    relative L2 and mean cosine similarity."""
    import torch
    B, H, N, d = q.shape
    g = torch.Generator(device="cpu").manual_seed(seed)
    rows = torch.randperm(N, generator=g)[:rows_per_head].to(q.device)
    num = den = 0.0
    worst = 0.0
    cos = []
    for b in range(B):
        for h in range(H):
            qs = q[b, h, rows].float()
            logits = (qs @ k[b, h].float().t()) * tau
            ref = torch.softmax(logits, dim=-1) @ v[b, h].float()
            got = out[b, h, rows].float()
            diff = got - ref
            worst = max(worst, float(diff.abs().max()))
            num += float((diff * diff).sum())
            den += float((ref * ref).sum())
            cos.append(torch.nn.functional.cosine_similarity(got, ref, dim=-1).mean().item())
    return {"max_abs": worst, "rel_l2": (num / den) ** 0.5, "mean_cos": sum(cos) / len(cos),
            "rows_per_head": int(rows.numel())}


def token_blocks(w, info, device):
    """Block of every raster token. Window layout: windows are numbered
    (frame, window row, window column) row-major over whole windows per
    frame. Packed edge windows (info.flags bit 0): the full windows are
    numbered that way among themselves; then a frame's partial windows
    (the right-hand column top to bottom, then the bottom row left to right,
    row-major inside each) form a stream over all frames, cut into blocks of
    win_h * win_w tokens."""
    import torch
    t = torch.arange(w.tokens, device=device)
    x = t % w.grid_w
    y = (t // w.grid_w) % w.grid_h
    f = t // (w.grid_w * w.grid_h)
    wy, wx = y // w.win_h, x // w.win_w
    if not (info.flags & 1):
        return (f * info.n_wy + wy) * info.n_wx + wx
    bs = w.win_h * w.win_w
    fwy, fwx = w.grid_h // w.win_h, w.grid_w // w.win_w
    rem_h, rem_w = w.grid_h - fwy * w.win_h, w.grid_w - fwx * w.win_w
    edge_frame = w.grid_h * w.grid_w - fwy * fwx * bs
    full = (wy < fwy) & (wx < fwx)
    right = fwy * w.win_h * rem_w
    in_right = (wy < fwy) & (wx >= fwx)
    pos_right = wy * w.win_h * rem_w + (y - wy * w.win_h) * rem_w + (x - fwx * w.win_w)
    ww = torch.clamp(w.grid_w - wx * w.win_w, max=w.win_w)
    pos_bottom = right + wx * rem_h * w.win_w + (y - fwy * w.win_h) * ww + (x - wx * w.win_w)
    pos = f * edge_frame + torch.where(in_right, pos_right, pos_bottom)
    return torch.where(full, (f * fwy + wy) * fwx + wx, info.n_full + pos // bs)


def fidelity(w, info, q, k, v, out, labels, scores, blocks_per_head, seed=0, blocks=None):
    """Error split and draft fidelity on a seeded sample of whole query blocks
    of every head, in fp32 against exact attention over the same bf16 inputs.

    Per sampled query block: dense attention (all keys), exact sparse
    attention (softmax over the retained blocks' keys only), and the true
    block mass M[i, j] (mean over block i's tokens of the dense probability
    on block j's keys). Reported: relative L2 over the sampled rows of
    sparse - dense (sparsification), out - sparse and out - dense (both over
    the dense norm); the mean over query blocks of the true mass on the hi,
    the lo and all retained blocks, and of the retained mass over the most
    any selection of that size keeps (recall); and the relative Frobenius
    distance between the draft scores C and M.

    labels: int8 [B*H, nb, nb] (device); scores: [B*H, nb, nb] draft scores C;
    blocks: the query blocks to sample (default: a seeded choice).
    """
    import torch
    B, H, N, d = q.shape
    nb = info.n_blocks
    dev = q.device
    tb = token_blocks(w, info, dev)
    if blocks is None:
        g = torch.Generator(device="cpu").manual_seed(seed)
        blocks = torch.randperm(nb, generator=g)[:blocks_per_head]
    blocks = torch.as_tensor(blocks).sort().values.to(dev)
    rows = torch.nonzero(torch.isin(tb, blocks)).flatten()
    pos = torch.searchsorted(blocks, tb[rows])                 # sampled-block slot of each row
    cnt = torch.zeros(len(blocks), device=dev).index_add_(0, pos, torch.ones(len(rows), device=dev))
    acc = dict(dense=0.0, sparse=0.0, q=0.0, total=0.0, cm=0.0, m=0.0)
    hi_m, lo_m, ret_m, rec = [], [], [], []
    for b in range(B):
        for h in range(H):
            bh = b * H + h
            kk, vv = k[b, h].float(), v[b, h].float()
            logits = (q[b, h, rows].float() @ kk.t()) * info.tau
            p = torch.softmax(logits, dim=-1)
            dense = p @ vv
            lab = labels[bh].to(dev)[blocks].long()            # [nS, nb]
            keep = lab[pos][:, tb] != 0                        # [R, N]
            sparse = torch.softmax(logits.masked_fill(~keep, float("-inf")), dim=-1) @ vv
            del logits, keep
            got = out[b, h, rows].float()
            acc["dense"] += float((dense * dense).sum())
            acc["sparse"] += float(((sparse - dense) ** 2).sum())
            acc["q"] += float(((got - sparse) ** 2).sum())
            acc["total"] += float(((got - dense) ** 2).sum())
            mrow = torch.zeros(len(rows), nb, device=dev).index_add_(1, tb, p)
            del p
            M = torch.zeros(len(blocks), nb, device=dev).index_add_(0, pos, mrow) / cnt[:, None]
            C = scores[bh].to(dev)[blocks].float()
            acc["cm"] += float(((C - M) ** 2).sum())
            acc["m"] += float((M * M).sum())
            n_ret = (lab != 0).sum(dim=1)
            best = torch.sort(M, dim=1, descending=True).values.cumsum(dim=1).gather(1, (n_ret - 1)[:, None])[:, 0]
            hi = (M * (lab == 2)).sum(dim=1)
            lo = (M * (lab == 1)).sum(dim=1)
            hi_m.append(hi)
            lo_m.append(lo)
            ret_m.append(hi + lo)
            rec.append((hi + lo) / best)
    mean = lambda xs: float(torch.cat(xs).mean())
    return {"sparsification_rel_l2": (acc["sparse"] / acc["dense"]) ** 0.5,
            "quantization_rel_l2": (acc["q"] / acc["dense"]) ** 0.5,
            "total_rel_l2": (acc["total"] / acc["dense"]) ** 0.5,
            "hi_mass": mean(hi_m), "lo_mass": mean(lo_m), "retained_mass": mean(ret_m),
            "recall": mean(rec), "draft_map_rel_fro": (acc["cm"] / acc["m"]) ** 0.5,
            "blocks_per_head": int(len(blocks)), "rows_per_head": int(len(rows))}


def sweep(args):
    import torch

    import block_sparse_mixed_amd as da2
    import synthetic as S
    base = S.WORKLOADS[args.workload]
    q, k, v = (t.to("cuda:0") for t in S.make_qkv(base))
    if args.pack_edges:
        base = dataclasses.replace(base, name=base.name + "-packed", pack_edges=True)
    for hi, lo in S.SWEEP_POINTS:
        w = S.with_budgets(base, hi, lo)
        cfg = da2.make_config(w.batch, w.heads, w.frames, w.grid_h, w.grid_w, w.head_dim, w.win_h, w.win_w,
                              w.budget_hi, w.budget_lo, out_dtype=da2.DA2_OUT_FP32,
                              flags=da2.DA2_FLAG_PACK_EDGES if w.pack_edges else 0)
        plan = da2.da2_plan(cfg)
        info = plan.info
        ws = plan.workspace(q.device)
        out = torch.empty(w.batch, w.heads, w.tokens, w.head_dim, dtype=torch.float32, device=q.device)
        stream = torch.cuda.current_stream(q.device)
        for _ in range(args.warmup):
            da2.da2_prepare(plan, q, k, v, ws, stream)
            da2.da2_attention(plan, ws, out, stream)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for _ in range(args.steps):
            da2.da2_prepare(plan, q, k, v, ws, stream)
        ev[1].record(stream)
        for _ in range(args.steps):
            da2.da2_attention(plan, ws, out, stream)
        ev[2].record(stream)
        torch.cuda.synchronize()
        prep_ms = ev[0].elapsed_time(ev[1]) / args.steps
        attn_ms = ev[1].elapsed_time(ev[2]) / args.steps
        dense, f_hi, f_lo = flops(w, info.n_blocks, info.n_hi, info.n_lo)
        t_star = f_hi / P_FP8 + f_lo / P_FP4
        err = dense_error(q, k, v, out, info.tau, args.sweep_rows)
        BH, nb = w.batch * w.heads, info.n_blocks
        labels = da2.workspace_section(plan, ws, "labels", torch.int8, (BH, nb, nb))
        scores = da2.workspace_section(plan, ws, "scores", torch.float64, (2, BH, nb, nb))[0]
        fid = fidelity(w, info, q, k, v, out, labels, scores, args.sweep_blocks)
        print(json.dumps({"sweep_point": {"budget_hi": hi, "budget_lo": lo, "n_hi": info.n_hi, "n_lo": info.n_lo},
                          "attention_ms": attn_ms, "prepare_ms": prep_ms,
                          "dense_equiv_tflops": dense / ((attn_ms + prep_ms) / 1e3) / 1e12,
                          "attention_executed_tflops": (f_hi + f_lo) / (attn_ms / 1e3) / 1e12,
                          "blended_roofline_frac": t_star / (attn_ms / 1e3) if f_hi + f_lo > 0 else None,
                          "error_vs_dense_fp32": err, "fidelity": fid, "workload": base.name}), flush=True)
        del ws, out, plan


def default_workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def time_layout(w, qd, kd, vd, pack, steps, warmup):
    """Plan the workload in one block layout and time `steps` whole steps
    (prepare + attention) on the current stream with HIP events, after
    `warmup` untimed ones. Returns the plan info, per-step prepare,
    attention and step times (ms) and the wall time of the timed loop (s)."""
    import torch

    import block_sparse_mixed_amd as da2
    cfg = da2.make_config(w.batch, w.heads, w.frames, w.grid_h, w.grid_w, w.head_dim, w.win_h, w.win_w,
                          w.budget_hi, w.budget_lo, out_dtype=da2.DA2_OUT_BF16,
                          flags=da2.DA2_FLAG_PACK_EDGES if pack else 0)
    plan = da2.da2_plan(cfg)
    ws = plan.workspace(qd.device)
    out = torch.empty(w.batch, w.heads, w.tokens, w.head_dim, dtype=torch.bfloat16, device=qd.device)
    stream = torch.cuda.current_stream(qd.device)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        da2.da2_prepare(plan, qd, kd, vd, ws, stream)
        if ev is not None:
            ev[1].record(stream)
        da2.da2_attention(plan, ws, out, stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    prep_ms = [e[0].elapsed_time(e[1]) for e in events]
    attn_ms = [e[1].elapsed_time(e[2]) for e in events]
    step_ms = [e[0].elapsed_time(e[2]) for e in events]
    nb = plan.info.n_blocks
    labels = da2.workspace_section(plan, ws, "labels", torch.int8, (w.batch * w.heads, nb, nb)).cpu()
    return plan.info, prep_ms, attn_ms, step_ms, wall, out, labels


def all_configs(args):
    """Every workload at its own budgets: step, preparation and attention
    times, throughput, roofline fraction and error vs dense fp32 (bf16
    output, the production path), and the oracle timed on the host over one
    head in full (unless --no-cpu-baseline)."""
    import torch

    import synthetic as S
    for name in ("tiny", "small", "wan480p", "hunyuan720p"):
        w = S.WORKLOADS[name]
        qc, kc, vc = S.make_qkv(w)
        q, k, v = (t.to("cuda:0") for t in (qc, kc, vc))
        info, prep_ms, attn_ms, step_ms, wall, out, _ = time_layout(w, q, k, v, False, args.steps, args.warmup)
        dense, f_hi, f_lo = flops(w, info.n_blocks, info.n_hi, info.n_lo)
        t_star = f_hi / P_FP8 + f_lo / P_FP4
        att_s = sum(attn_ms) / len(attn_ms) / 1e3
        step_s = sum(step_ms) / len(step_ms) / 1e3
        err = dense_error(q, k, v, out, info.tau, args.error_rows)
        cpu = None
        if not args.no_cpu_baseline:
            cpu = cpu_baseline(w, qc, kc, vc, 1, args.cpu_workers or default_workers())
        print(json.dumps({"workload": name, "n_blocks": info.n_blocks, "n_hi": info.n_hi, "n_lo": info.n_lo,
                          "attention_ms": att_s * 1e3, "attention_ms_min": min(attn_ms),
                          "prepare_ms": sum(prep_ms) / len(prep_ms), "step_ms_events": step_s * 1e3,
                          "dense_equiv_tflops_step": dense / step_s / 1e12,
                          "attention_executed_tflops": (f_hi + f_lo) / att_s / 1e12,
                          "blended_roofline_frac": t_star / att_s,
                          "error_vs_dense_fp32": err, "cpu_baseline": cpu}), flush=True)
        del q, k, v, out
        torch.cuda.empty_cache()


def dit_block(args):
    """The attention sublayer of a video DiT block at the workload's shape,
    hidden size heads x head_dim, random bf16 weights (timing only):
      fused   x -> QKV projection -> da2::attention_qkv reading the projection
              output in place -> output projection reading the op's
              [B, N, H, d] output in place;
      unfused the same projections and library call with the usual layout
              changes around the attention: split + permute of the QKV
              output to contiguous [B, H, N, d], and the output back to
              [B, N, H*d];
      dense   the same projections around torch's scaled_dot_product_attention
              (bf16, dense) on the permuted q, k, v.
    Prints one JSON line with the per-step milliseconds of each."""
    import torch
    import torch.nn.functional as Fn

    import block_sparse_mixed_amd as da2
    import synthetic as S
    from block_sparse_mixed_amd import torch_op
    w = S.WORKLOADS[args.workload]
    B, H, d, N = w.batch, w.heads, w.head_dim, w.tokens
    C = H * d
    torch.manual_seed(0)
    m = torch_op.DA2SelfAttention(C, H, w.frames, w.grid_h, w.grid_w, win=(w.win_h, w.win_w),
                                  budget_hi=w.budget_hi, budget_lo=w.budget_lo,
                                  flags=da2.DA2_FLAG_PACK_EDGES if args.pack_edges else 0, device="cuda")
    x = torch.randn(B, N, C, device="cuda", dtype=torch.bfloat16)
    grid = (w.frames, w.grid_h, w.grid_w, w.win_h, w.win_w, w.budget_hi, w.budget_lo)

    def fused():
        return m(x)

    def split():
        qkv = m.qkv(x).view(B, N, 3, H, d).permute(2, 0, 3, 1, 4).contiguous()
        return qkv[0], qkv[1], qkv[2]

    def unfused():
        q, k, v = split()
        o = da2.attention(q, k, v, *grid, out_dtype=torch.bfloat16, flags=m.flags)
        return m.proj(o.transpose(1, 2).reshape(B, N, C))

    def dense():
        q, k, v = split()
        o = Fn.scaled_dot_product_attention(q, k, v)
        return m.proj(o.transpose(1, 2).reshape(B, N, C))

    def projections():
        return m.proj(m.qkv(x)[..., :C].contiguous())

    res = {"dit_block": {"workload": w.name, "hidden": C, "heads": H, "tokens": N, "batch": B,
                         "budget_hi": w.budget_hi, "budget_lo": w.budget_lo,
                         "layout": "packed_edges" if args.pack_edges else "padded_windows"}}
    with torch.no_grad():
        for name, fn in (("fused", fused), ("unfused", unfused), ("dense_sdpa", dense),
                         ("projections_only", projections)):
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            res[name + "_ms"] = e0.elapsed_time(e1) / args.steps
        y_fused, y_unfused = fused(), unfused()
        torch.cuda.synchronize()
        res["fused_equals_unfused"] = bool(torch.equal(y_fused, y_unfused))
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.sweep:
        sweep(args)
        return
    if args.all_configs:
        all_configs(args)
        return
    if args.dit_block:
        dit_block(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards over heads with no communication; see the design notes).", file=sys.stderr)
        sys.exit(2)
    import torch

    import block_sparse_mixed_amd as da2
    import synthetic as S

    w = S.WORKLOADS[args.workload]
    q, k, v = S.make_qkv(w)
    if args.budgets:
        w = S.with_budgets(w, *args.budgets)
    if args.pack_edges:
        w = dataclasses.replace(w, name=w.name + "-packed", pack_edges=True)
    cpu = None
    if not args.no_cpu_baseline:
        workers = args.cpu_workers or default_workers()
        cpu = cpu_baseline(w, q, k, v, min(args.cpu_heads, w.batch * w.heads), workers)
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    info, prep_ms, attn_ms, step_ms, wall, out, labels = time_layout(w, qd, kd, vd, args.pack_edges, args.steps,
                                                                     args.warmup)
    err = dense_error(qd, kd, vd, out, info.tau, args.error_rows)
    del out
    alt = None
    if not args.no_alt_layout:
        a_info, a_prep, a_attn, a_step, _, a_out, _ = time_layout(w, qd, kd, vd, not args.pack_edges, args.steps,
                                                                  args.warmup)
        a_err = dense_error(qd, kd, vd, a_out, a_info.tau, args.error_rows)
        del a_out
        a_dense, a_hi, a_lo = flops(w, a_info.n_blocks, a_info.n_hi, a_info.n_lo)
        a_attn_s = sum(a_attn) / len(a_attn) / 1e3
        a_step_s = sum(a_step) / len(a_step) / 1e3
        alt = {"layout": "packed_edges" if not args.pack_edges else "padded_windows",
               "n_blocks": a_info.n_blocks, "n_hi": a_info.n_hi, "n_lo": a_info.n_lo,
               "attention_ms": a_attn_s * 1e3, "prepare_ms": sum(a_prep) / len(a_prep),
               "step_ms_events": a_step_s * 1e3,
               "dense_equiv_tflops_step_events": a_dense / a_step_s / 1e12,
               "roofline_frac": (a_hi / P_FP8 + a_lo / P_FP4) / a_attn_s,
               "error_vs_dense_fp32": a_err}
    ms_per_step = wall * 1e3 / args.steps
    dense, f_hi, f_lo = flops(w, info.n_blocks, info.n_hi, info.n_lo)
    t_star = f_hi / P_FP8 + f_lo / P_FP4
    blended_peak = (f_hi + f_lo) / t_star
    attn_avg_s = sum(attn_ms) / len(attn_ms) / 1e3
    achieved = (f_hi + f_lo) / attn_avg_s
    # the instructions actually issued: half of F_hi (QK^T) on bf16 MFMAs
    t_star_instr = 0.5 * f_hi / P_BF16 + 0.5 * f_hi / P_FP8 + f_lo / P_FP4
    r_hi, r_lo = real_slot_flops(w, info, labels)
    res = {
        "metric": METRIC,
        "value": dense / (ms_per_step / 1e3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8+mxfp4",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "frames": w.frames,
                   "grid": [w.grid_h, w.grid_w], "tokens": w.tokens, "head_dim": w.head_dim,
                   "window": [w.win_h, w.win_w], "budget_hi": w.budget_hi, "budget_lo": w.budget_lo,
                   "n_blocks": info.n_blocks, "n_hi": info.n_hi, "n_lo": info.n_lo, "out_dtype": "bf16",
                   "layout": "packed_edges" if args.pack_edges else "padded_windows"},
        "roofline": {"bound": "mfma", "achieved": achieved / 1e12, "peak": blended_peak / 1e12, "unit": "TFLOP/s",
                     "frac": achieved / blended_peak, "traffic": recorded_traffic(w.name)},
        "cpu_baseline": cpu,
        "error_vs_dense_fp32": err,
        "attention_ms": sum(attn_ms) / len(attn_ms),
        "attention_ms_min": min(attn_ms),
        "prepare_ms": sum(prep_ms) / len(prep_ms),
        "step_ms_events": sum(step_ms) / len(step_ms),
        "attention_dense_equiv_tflops": dense / attn_avg_s / 1e12,
        "attention_executed_tflops": achieved / 1e12,
        "blended_roofline_ms": t_star * 1e3,
        "issued_mix_roofline_ms": t_star_instr * 1e3,
        "flops": {"dense_equiv": dense, "f_hi": f_hi, "f_lo": f_lo},
        "real_slots": {"f_hi": r_hi, "f_lo": r_lo, "useful_fraction": (r_hi + r_lo) / (f_hi + f_lo),
                       "attention_tflops": (r_hi + r_lo) / attn_avg_s / 1e12},
        "other_layout": alt,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
