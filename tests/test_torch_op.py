"""The torch custom op around the path: registration, fake (meta) shapes,
argument checks, and the separate output strides of the C ABI. No GPU."""

import pytest
import torch

import block_sparse_mixed_amd as da2
from block_sparse_mixed_amd import torch_op  # noqa: F401  (registers da2::attention_qkv)


def test_op_is_registered_with_a_fake_implementation():
    from torch._subclasses.fake_tensor import FakeTensorMode
    with FakeTensorMode():
        qkv = torch.empty(2, 2 * 16 * 16, 3, 4, 64, dtype=torch.bfloat16)
        out = torch.ops.da2.attention_qkv(qkv, 2, 16, 16, 4, 4, 0.25, 0.25)
    assert tuple(out.shape) == (2, 512, 4, 64) and out.dtype == torch.bfloat16


def test_op_rejects_bad_arguments_before_the_library():
    good = torch.zeros(1, 2 * 8 * 8, 3, 2, 32, dtype=torch.bfloat16)
    args = (2, 8, 8, 4, 4, 0.25, 0.25)
    with pytest.raises(ValueError, match=r"\[B, N, 3, H, d\]"):
        torch.ops.da2.attention_qkv(good[:, :, :2], *args)
    with pytest.raises(ValueError, match="bfloat16"):
        torch.ops.da2.attention_qkv(good.float(), *args)
    with pytest.raises(ValueError, match="latent grid"):
        torch.ops.da2.attention_qkv(good, 1, 8, 8, 4, 4, 0.25, 0.25)
    with pytest.raises(ValueError, match="GPU"):
        torch.ops.da2.attention_qkv(good, *args)


def test_module_projections_have_the_dit_shapes():
    m = torch_op.DA2SelfAttention(256, 2, 2, 8, 8, win=(4, 4), device="cpu")
    assert m.qkv.weight.shape == (768, 256) and m.proj.weight.shape == (256, 256)
    with pytest.raises(ValueError):
        torch_op.DA2SelfAttention(250, 3, 2, 8, 8)


def _cfg(**kw):
    base = dict(batch=1, heads=12, frames=21, grid_h=30, grid_w=52, head_dim=128, win_h=8, win_w=16,
                budget_hi=0.15, budget_lo=0.35)
    base.update(kw)
    return da2.make_config(**base)


def test_plan_output_strides():
    n = 32760
    # a fused [B, N, 3, H, d] input and a [B, N, H, d] output
    fused = (n * 3 * 12 * 128, 128, 3 * 12 * 128)
    bnhd = (n * 12 * 128, 128, 12 * 128)
    da2.da2_plan(_cfg(strides=fused, out_strides=bnhd))
    for bad in ((-1, 128, 1536), (n * 1536, 128, 64), (0, 128, 1536)):
        with pytest.raises(da2.Da2Error) as e:
            da2.da2_plan(_cfg(strides=fused, out_strides=bad))
        assert e.value.status == da2.DA2_ERR_INVALID_ARG
    # the output strides follow the vector rule on their own: checked by
    # da2_attention before anything is enqueued
    fake, big = 1 << 20, 1 << 40
    p = da2.da2_plan(_cfg(strides=fused, out_strides=(n * 1540, 128, 1540)))
    assert da2._lib.da2_attention(p.handle, fake, big, fake, None) == da2.DA2_ERR_UNSUPPORTED
