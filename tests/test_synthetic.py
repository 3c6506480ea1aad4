"""The seeded input generator: shapes, determinism and the stated statistics."""

import numpy as np
import torch

import synthetic as S


def test_shapes_dtype_and_determinism():
    q, k, v = S.make_qkv(S.TINY)
    assert q.shape == (1, 1, 512, 64) and q.dtype == torch.bfloat16
    q2, k2, v2 = S.make_qkv(S.TINY)
    assert torch.equal(q, q2) and torch.equal(k, k2) and torch.equal(v, v2)
    assert not torch.equal(q, k)


def test_fields_are_smooth_and_v_is_standard_normal():
    q, k, v = S.make_qkv(S.SMALL)
    x = q[0, 0].float().reshape(5, 32, 32, 128)
    # neighbouring tokens are strongly correlated (smooth field), far ones are not
    a, b, c = x[:, :, :-1], x[:, :, 1:], x.roll(16, dims=2)
    near = torch.corrcoef(torch.stack([a.flatten(), b.flatten()]))[0, 1]
    far = torch.corrcoef(torch.stack([x.flatten(), c.flatten()]))[0, 1]
    assert near > 0.8 and far < near
    vv = v.float()
    assert abs(vv.mean().item()) < 0.01 and abs(vv.std().item() - 1) < 0.01


def test_outlier_channels_small():
    q, k, _ = S.make_qkv(S.SMALL)
    s = q[0].float().abs().mean(dim=(0, 1))
    top = torch.topk(s, 3).values
    assert top[1] > 4 * top[2]                    # exactly two channels stand out
    sk = k[0].float().abs().mean(dim=(0, 1))
    assert set(torch.topk(s, 2).indices.tolist()) == set(torch.topk(sk, 2).indices.tolist())
