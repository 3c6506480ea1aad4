"""The path as one torch custom op between a DiT block's QKV projection and
its output projection.

[DraftAttention (arXiv 2505.14708), abstract]: the method replaces the
attention call of a video diffusion transformer without retraining; tokens are
reordered into windows for the computation and the original order is restored
afterwards. [DraftAttention news article, method step 5]: plug-and-play in
HunyuanVideo and Wan2.1.

``torch.ops.da2.attention_qkv(qkv, ...)`` takes the fused QKV projection
output as it comes out of the projection GEMM, ``[B, N, 3, H, d]`` (a view of
``[B, N, 3*H*d]``), and hands q, k, v to the library as strided views: the
operand preparation kernel gathers each window's rows straight from it, so
there is no split, permute or copy in front of the attention. The attention
kernel writes every output row straight to its raster position in
``[B, N, H, d]`` (separate output strides), which viewed as ``[B, N, H*d]`` is
the output projection's input: no transpose or copy behind it either.

Argument marshalling only; the library does all the work. The op has a fake
(meta) implementation, so it traces under torch.compile / torch.export. It
has no autograd formula (the path is an inference path).
"""

from __future__ import annotations

import torch

import block_sparse_mixed_amd as da2

_PLANS: dict = {}


def _plan(key):
    p = _PLANS.get(key)
    if p is None:
        (B, H, frames, grid_h, grid_w, d, win_h, win_w, budget_hi, budget_lo, softmax_scale, flags,
         strides, out_strides) = key
        cfg = da2.make_config(B, H, frames, grid_h, grid_w, d, win_h, win_w, budget_hi, budget_lo, softmax_scale,
                              strides=strides, out_dtype=da2.DA2_OUT_BF16, flags=flags, out_strides=out_strides)
        p = da2.da2_plan(cfg)
        _PLANS[key] = p
    return p


def _check(qkv: torch.Tensor, frames: int, grid_h: int, grid_w: int):
    if qkv.dim() != 5 or qkv.shape[2] != 3:
        raise ValueError(f"qkv must be [B, N, 3, H, d], got {tuple(qkv.shape)}")
    if qkv.dtype != torch.bfloat16:
        raise ValueError("qkv must be bfloat16")
    B, N, _, H, d = qkv.shape
    if N != frames * grid_h * grid_w:
        raise ValueError(f"qkv has {N} tokens, but a {frames} x {grid_h} x {grid_w} latent grid has "
                         f"{frames * grid_h * grid_w}")
    if qkv.stride(4) != 1:
        raise ValueError("the last dimension of qkv must be contiguous")


@torch.library.custom_op("da2::attention_qkv", mutates_args=())
def attention_qkv(qkv: torch.Tensor, frames: int, grid_h: int, grid_w: int, win_h: int, win_w: int,
                  budget_hi: float, budget_lo: float, softmax_scale: float = 0.0, flags: int = 0) -> torch.Tensor:
    """Draft-guided fp8/MXFP4 block-sparse attention of a fused QKV tensor
    ``[B, N, 3, H, d]`` (bf16, tokens in raster order of a frames x grid_h x
    grid_w latent grid); returns ``[B, N, H, d]`` bf16 in the same token
    order. Budgets, window and flags as in ``da2_config``."""
    _check(qkv, frames, grid_h, grid_w)
    if qkv.device.type != "cuda":
        raise ValueError("qkv must be on a GPU")
    B, N, _, H, d = qkv.shape
    q, k, v = (qkv[:, :, i].transpose(1, 2) for i in range(3))          # [B, H, N, d] views
    out = torch.empty(B, N, H, d, dtype=torch.bfloat16, device=qkv.device)
    o = out.transpose(1, 2)                                             # [B, H, N, d] view
    key = (B, H, frames, grid_h, grid_w, d, win_h, win_w, float(budget_hi), float(budget_lo), float(softmax_scale),
           int(flags), tuple(q.stride()[:3]), tuple(o.stride()[:3]))
    plan = _plan(key)
    # no clearing needed: preparation writes every workspace byte attention reads
    ws = torch.empty(int(plan.info.workspace_bytes), dtype=torch.uint8, device=qkv.device)
    stream = torch.cuda.current_stream(qkv.device)
    da2.da2_prepare(plan, q, k, v, ws, stream)
    da2.da2_attention(plan, ws, o, stream)
    return out


@attention_qkv.register_fake
def _attention_qkv_fake(qkv, frames, grid_h, grid_w, win_h, win_w, budget_hi, budget_lo, softmax_scale=0.0,
                        flags=0):
    _check(qkv, frames, grid_h, grid_w)
    B, N, _, H, d = qkv.shape
    return qkv.new_empty((B, N, H, d))


class DA2SelfAttention(torch.nn.Module):
    """The attention sublayer of a video DiT block: QKV projection, the
    DraftAttention2 path (``da2::attention_qkv``), output projection. The
    token sequence is a frames x grid_h x grid_w latent grid in raster order."""

    def __init__(self, dim: int, heads: int, frames: int, grid_h: int, grid_w: int, win=(8, 16),
                 budget_hi: float = 0.15, budget_lo: float = 0.35, flags: int = 0, bias: bool = True,
                 device=None, dtype=torch.bfloat16):
        super().__init__()
        if dim % heads:
            raise ValueError("dim must be a multiple of heads")
        self.heads = heads
        self.grid = (frames, grid_h, grid_w)
        self.win = tuple(win)
        self.budgets = (float(budget_hi), float(budget_lo))
        self.flags = int(flags)
        self.qkv = torch.nn.Linear(dim, 3 * dim, bias=bias, device=device, dtype=dtype)
        self.proj = torch.nn.Linear(dim, dim, bias=bias, device=device, dtype=dtype)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        B, N, C = x.shape
        qkv = self.qkv(x).view(B, N, 3, self.heads, C // self.heads)
        o = torch.ops.da2.attention_qkv(qkv, *self.grid, *self.win, *self.budgets, 0.0, self.flags)
        return self.proj(o.view(B, N, C))
