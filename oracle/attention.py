"""Block-sparse mixed-precision attention with phases that share softmax state.

[DA2] abstract: one attention kernel has a phase per precision; the phases
share data movement, the softmax statistics and the output accumulator; the
higher-precision (8-bit) phase covers the top-ranked blocks and the
lower-precision (4-bit) phase the other retained blocks; skipped blocks are
not computed. [DA1] abstract: outputs go back to the original token order.

Readings (the pages give no formula), for a real query token r of block i
with retained key blocks R = HI(i) u LO(i):
* s_rj = dequant(q_r) . dequant(k_j), with the fp8 operands in HI blocks and
  the MXFP4 operands in LO blocks; padded key slots are excluded.
* Base-2 softmax with an integer shift: x = s * tau * log2(e),
  m_r = ceil(max_j x_rj), p = 2^(x - m_r) in (0, 1].
* The probabilities enter the PV product in the phase's own format:
  HI: P~ = E4M3(p * 2^8) * 2^-8 (RNE);
  LO: P~ = MXFP4 of p over groups of 32 consecutive key slots of the key
  block (padded keys carry p = 0), scale from shared_exponent(amax, 6).
  Power-of-two shifts of p leave both encodings unchanged (apart from E4M3
  subnormals), so a GPU that applies its running integer max gets the same
  P~ as this final-max definition.
* Normaliser l = sum of P~, so the applied weights sum to exactly one.
* O_r = sum_j P~_rj V~_j / l_r, with V~ the fp8 or MXFP4 dequantized values
  according to the key block's phase.
"""

from __future__ import annotations

import numpy as np

from .draft import HI, LO
from .formats import decode_e4m3, encode_e4m3
from .quant import dequant_mx_lastaxis, quantize_mx_lastaxis

LOG2E = 1.0 / np.log(2.0)
P8_SHIFT = 8


def quantize_p_hi(p: np.ndarray) -> np.ndarray:
    return decode_e4m3(encode_e4m3(p * 2.0 ** P8_SHIFT)) * 2.0 ** -P8_SHIFT


def quantize_p_lo(p: np.ndarray) -> np.ndarray:
    """p [..., bs_k] along one key block's slots -> MXFP4-quantized values."""
    codes, e = quantize_mx_lastaxis(p)
    return dequant_mx_lastaxis(codes, e)


def attend_block(i: int, labels_row: np.ndarray, ops: dict, valid: np.ndarray, tau: float,
                 quantize: bool = True, return_weights: bool = False):
    """Outputs [bs, d] float64 for the slots of query block i (padded rows are NaN).

    ops: the dict from quant.prepare_operands plus "q", "k", "v" raw blocks
    ([n_b, bs, d] float64) for the quantize=False path (a test-only switch that
    replaces every quantizer by the identity).
    """
    hi = np.flatnonzero(labels_row == HI)
    lo = np.flatnonzero(labels_row == LO)
    if quantize:
        q_hi, q_lo = ops["q8_deq"][i], ops["q4_deq"][i]
        k_hi, k_lo = ops["k8_deq"][hi], ops["k4_deq"][lo]
        v_hi, v_lo = ops["v8_deq"][hi], ops["v4_deq"][lo]
    else:
        q_hi = q_lo = ops["q"][i]
        k_hi, k_lo = ops["k"][hi], ops["k"][lo]
        v_hi, v_lo = ops["v"][hi], ops["v"][lo]
    c = tau * LOG2E
    x_hi = np.einsum("sd,jtd->sjt", q_hi, k_hi) * c          # [bs_q, n_hi, bs_k]
    x_lo = np.einsum("sd,jtd->sjt", q_lo, k_lo) * c
    x_hi = np.where(valid[hi][None], x_hi, -np.inf)
    x_lo = np.where(valid[lo][None], x_lo, -np.inf)
    row_max = np.maximum(x_hi.max(axis=(1, 2), initial=-np.inf), x_lo.max(axis=(1, 2), initial=-np.inf))
    m = np.ceil(row_max)
    p_hi = np.exp2(x_hi - m[:, None, None])
    p_lo = np.exp2(x_lo - m[:, None, None])
    if quantize:
        P_hi = quantize_p_hi(p_hi)
        P_lo = quantize_p_lo(p_lo)
    else:
        P_hi, P_lo = p_hi, p_lo
    num = np.einsum("sjt,jtd->sd", P_hi, v_hi) + np.einsum("sjt,jtd->sd", P_lo, v_lo)
    den = P_hi.sum(axis=(1, 2)) + P_lo.sum(axis=(1, 2))
    out = num / den[:, None]
    out[~valid[i]] = np.nan
    if return_weights:
        nb, bs = labels_row.shape[0], valid.shape[1]
        w = np.zeros((valid.shape[1], nb, bs))
        w[:, hi] = P_hi / den[:, None, None]
        w[:, lo] = P_lo / den[:, None, None]
        return out, w
    return out
