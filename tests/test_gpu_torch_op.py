"""GPU tests of the torch custom op da2::attention_qkv (MI355X only): it is
argument marshalling around the library, so its output equals the library's
on the same values bit for bit, in the [B, N, H, d] layout the output
projection reads."""

import dataclasses

import pytest
import torch

import synthetic as S

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_sparse_mixed_amd as da2
    from block_sparse_mixed_amd import torch_op
    return da2, torch_op


def _say(*a):
    print("[gpu]", *a, flush=True)


@pytest.mark.parametrize("pack", [False, True])
def test_op_equals_the_library_on_the_same_values(ops, pack):
    da2, _ = ops
    w = dataclasses.replace(S.SMALL, name="small-b2", batch=2)
    q, k, v = (t.cuda() for t in S.make_qkv(w))
    qkv = torch.stack([t.transpose(1, 2) for t in (q, k, v)], dim=2).contiguous()   # [B, N, 3, H, d]
    flags = da2.DA2_FLAG_PACK_EDGES if pack else 0
    args = (w.frames, w.grid_h, w.grid_w, w.win_h, w.win_w, w.budget_hi, w.budget_lo)
    _say(f"da2::attention_qkv small batch 2, pack={pack}")
    out = torch.ops.da2.attention_qkv(qkv, *args, 0.0, flags)
    ref = da2.attention(q, k, v, *args, out_dtype=torch.bfloat16, flags=flags)      # [B, H, N, d]
    torch.cuda.synchronize()
    assert out.shape == (w.batch, w.tokens, w.heads, w.head_dim) and out.is_contiguous()
    assert torch.equal(out, ref.transpose(1, 2))


def test_self_attention_module_is_the_composition(ops):
    _, torch_op = ops
    w = S.SMALL
    torch.manual_seed(0)
    dim = w.heads * w.head_dim
    m = torch_op.DA2SelfAttention(dim, w.heads, w.frames, w.grid_h, w.grid_w, win=(w.win_h, w.win_w),
                                  budget_hi=w.budget_hi, budget_lo=w.budget_lo, device="cuda")
    x = torch.randn(1, w.tokens, dim, device="cuda", dtype=torch.bfloat16)
    _say("DA2SelfAttention forward (small)")
    with torch.no_grad():
        y = m(x)
        qkv = m.qkv(x).view(1, w.tokens, 3, w.heads, w.head_dim)
        o = torch.ops.da2.attention_qkv(qkv, w.frames, w.grid_h, w.grid_w, w.win_h, w.win_w, w.budget_hi,
                                        w.budget_lo)
        y2 = m.proj(o.reshape(1, w.tokens, dim))
    torch.cuda.synchronize()
    assert torch.isfinite(y).all() and torch.equal(y, y2)


def test_opcheck_schema_and_fake(ops):
    w = S.TINY
    q, k, v = (t.cuda() for t in S.make_qkv(w))
    qkv = torch.stack([t.transpose(1, 2) for t in (q, k, v)], dim=2).contiguous()
    _say("opcheck da2::attention_qkv (tiny)")
    torch.library.opcheck(torch.ops.da2.attention_qkv.default,
                          (qkv, w.frames, w.grid_h, w.grid_w, w.win_h, w.win_w, w.budget_hi, w.budget_lo, 0.0, 0),
                          test_utils=("test_schema", "test_faketensor"))
