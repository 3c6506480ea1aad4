"""Operand quantization: fp8 E4M3 per block, MXFP4 per 32-element group.

[DA2] abstract: operands are prepared in one fused pass for the 8-bit and the
4-bit phases. The formats and scale codes follow [OFP8] and [OCP-MX].

Readings:
* fp8: one power-of-two scale per (tensor, head, block) over all of the
  block's values (padded slots are zero), e = shared_exponent(amax, 448).
* MXFP4: groups of 32 consecutive elements along the contraction axis of the
  product the operand enters: Q and K along the head dimension (per token);
  V along the block's slots (per channel), since PV contracts over keys.
  A block of fewer than 32 slots forms one group, zero-padded.
* Codes are RNE(x * 2^-e); |x * 2^-e| never exceeds the format maximum by the
  choice of e, so no value saturates.
"""

from __future__ import annotations

import numpy as np

from .formats import (E2M1_MAX, E4M3_MAX, decode_e2m1, decode_e4m3, encode_e2m1,
                      encode_e4m3, shared_exponent)

MX_GROUP = 32


def quantize_fp8_block(tile: np.ndarray):
    """tile [..., bs, d] float64 -> (codes uint8 same shape, exponent int per leading index)."""
    amax = np.abs(tile).reshape(tile.shape[:-2] + (-1,)).max(axis=-1)
    e = shared_exponent(amax, E4M3_MAX)
    scaled = tile * np.ldexp(1.0, -e)[..., None, None]
    return encode_e4m3(scaled), e


def dequant_fp8_block(codes: np.ndarray, e) -> np.ndarray:
    return decode_e4m3(codes) * np.ldexp(1.0, np.asarray(e))[..., None, None]


def quantize_mx_lastaxis(x: np.ndarray):
    """Groups of 32 along the last axis (zero-padded to a multiple of 32).

    Returns (codes uint8 [..., L], exponents int [..., ceil(L/32)]).
    """
    L = x.shape[-1]
    G = -(-L // MX_GROUP)
    pad = G * MX_GROUP - L
    xp = np.concatenate([x, np.zeros(x.shape[:-1] + (pad,))], axis=-1) if pad else x
    grp = xp.reshape(x.shape[:-1] + (G, MX_GROUP))
    amax = np.abs(grp).max(axis=-1)
    e = shared_exponent(amax, E2M1_MAX)
    codes = encode_e2m1(grp * np.ldexp(1.0, -e)[..., None])
    return codes.reshape(xp.shape)[..., :L], e


def dequant_mx_lastaxis(codes: np.ndarray, e: np.ndarray) -> np.ndarray:
    L = codes.shape[-1]
    scale = np.repeat(np.ldexp(1.0, e), MX_GROUP, axis=-1)[..., :L]
    return decode_e2m1(codes) * scale


def prepare_operands(qb: np.ndarray, kb: np.ndarray, vb: np.ndarray) -> dict:
    """Block-gathered [n_b, bs, d] float64 Q/K/V -> codes, exponents, dequantized values."""
    out = {}
    for name, t in (("q", qb), ("k", kb), ("v", vb)):
        c8, e8 = quantize_fp8_block(t)
        out[name + "8"] = c8
        out[name + "8_exp"] = e8
        out[name + "8_deq"] = dequant_fp8_block(c8, e8)
    for name, t in (("q", qb), ("k", kb)):
        c4, e4 = quantize_mx_lastaxis(t)               # along d, per token
        out[name + "4"] = c4
        out[name + "4_exp"] = e4
        out[name + "4_deq"] = dequant_mx_lastaxis(c4, e4)
    vt = np.swapaxes(vb, -1, -2)                       # [n_b, d, bs]: groups along slots
    c4, e4 = quantize_mx_lastaxis(vt)
    out["v4t"] = c4
    out["v4t_exp"] = e4
    out["v4_deq"] = np.swapaxes(dequant_mx_lastaxis(c4, e4), -1, -2)
    return out
