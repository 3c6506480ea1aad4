"""GPU test of the entry point that allocates nothing (da2_forward_scratch):
its output equals that of da2_prepare + da2_attention on a caller's
workspace, bit for bit, over two calls in a row, the second one smaller (the
static workspace then still holds the first call's bytes)."""

import dataclasses

import pytest
import torch

import synthetic as S

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu]", *a, flush=True)


def _cfg(da2, w):
    return da2.make_config(w.batch, w.heads, w.frames, w.grid_h, w.grid_w, w.head_dim, w.win_h, w.win_w,
                           w.budget_hi, w.budget_lo, out_dtype=da2.DA2_OUT_FP32,
                           flags=da2.DA2_FLAG_PACK_EDGES if w.pack_edges else 0)


def test_forward_scratch_matches_prepare_attention_on_two_calls():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_sparse_mixed_amd as da2
    first = dataclasses.replace(S.WAN480, name="wan480p-6heads", heads=6)      # 197 MiB of the 256 MiB
    second = S.SMALL
    for w in (first, second):
        plan = da2.da2_plan(_cfg(da2, w))
        assert plan.info.workspace_bytes <= da2.SCRATCH_BYTES
        q, k, v = (t.cuda() for t in S.make_qkv(w))
        shape = (w.batch, w.heads, w.tokens, w.head_dim)
        # the reference: the existing pair, on a workspace filled with 0xFF
        # bytes (NaN codes and scales): prepare writes every byte attention reads
        ws = torch.full((int(plan.info.workspace_bytes),), 255, dtype=torch.uint8, device="cuda")
        want = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
        _say(f"da2_prepare + da2_attention {w.name} ({plan.info.workspace_bytes / 2**20:.0f} MiB)")
        da2.da2_prepare(plan, q, k, v, ws)
        da2.da2_attention(plan, ws, want)
        got = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
        _say(f"da2_forward_scratch {w.name}")
        da2.da2_forward_scratch(plan, q, k, v, got)
        torch.cuda.synchronize()
        assert torch.isfinite(want).all()
        assert torch.equal(got, want), f"{w.name}: static-workspace output differs"
        del ws, want, got, q, k, v
