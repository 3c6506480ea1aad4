"""Pins for oracle.formats / oracle.quant against the format definitions and torch."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import quant as Q


def test_e4m3_table_matches_torch_float8():
    torch_vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    same = (torch_vals == F.E4M3_VALUES) | (np.isnan(torch_vals) & np.isnan(F.E4M3_VALUES))
    assert same.all()


def test_e4m3_landmarks():
    # OFP8 E4M3: max 448, min normal 2^-6, min subnormal 2^-9, 1.0 at exponent field 7
    assert F.E4M3_VALUES[0x7E] == 448.0
    assert F.E4M3_VALUES[0x08] == 2.0 ** -6
    assert F.E4M3_VALUES[0x01] == 2.0 ** -9
    assert F.E4M3_VALUES[0x38] == 1.0
    assert np.isnan(F.E4M3_VALUES[0x7F]) and np.isnan(F.E4M3_VALUES[0xFF])
    assert F.E4M3_VALUES[0x80] == 0.0 and np.signbit(F.E4M3_VALUES[0x80])


def test_e2m1_table_is_the_mx_set():
    mags = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(F.E2M1_VALUES[:8]) == mags
    assert list(-F.E2M1_VALUES[8:]) == mags


def _all_bf16_values_in(limit):
    bits = np.arange(65536, dtype=np.uint32) << 16
    v = bits.view(np.float32).astype(np.float64)
    return v[np.isfinite(v) & (np.abs(v) <= limit)]


def test_encode_e4m3_matches_torch_exhaustive_bf16():
    v = _all_bf16_values_in(448.0)
    for shift in (0, -3, 5):                 # also move values across the subnormal range
        x = np.ldexp(v, shift)
        x = x[np.abs(x) <= 448.0]
        ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        got = F.encode_e4m3(x)
        # torch keeps the sign of zero results too
        assert np.array_equal(got, ref)


def test_encode_e4m3_ties_to_even():
    # midpoints between consecutive positive codes: must land on the even code
    vals = F.E4M3_VALUES[:0x7F]
    mids = 0.5 * (vals[:-1] + vals[1:])
    codes = F.encode_e4m3(mids)
    assert np.all(codes % 2 == 0)
    assert np.all((codes == np.arange(0x7E)) | (codes == np.arange(1, 0x7F)))
    ref = torch.from_numpy(mids).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


def test_encode_e2m1_midpoints_hand_derived():
    # tie cases decided by hand from RNE on {0,.5,1,1.5,2,3,4,6}
    cases = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6,
             0.26: 1, 0.74: 1, 1.3: 3, 2.6: 5, 5.01: 7, 6.0: 7, 0.0: 0}
    for x, c in cases.items():
        assert F.encode_e2m1([x])[0] == c, x
        assert F.encode_e2m1([-x])[0] == c | 8, x


def test_encode_roundtrip_and_monotone():
    for table, enc, n in ((F.E4M3_VALUES, F.encode_e4m3, 0x7F), (F.E2M1_VALUES, F.encode_e2m1, 8)):
        codes = np.arange(n)
        assert np.array_equal(enc(table[codes]), codes)
        x = np.linspace(0, table[n - 1], 20001)
        c = enc(x).astype(int)
        assert np.all(np.diff(table[c]) >= 0)
        # error never exceeds half the local spacing
        err = np.abs(table[c] - x)
        up = np.minimum(c + 1, n - 1)
        down = np.maximum(c - 1, 0)
        half = 0.5 * np.maximum(table[up] - table[c], table[c] - table[down])
        assert np.all(err <= half + 1e-15)


def _smallest_exponent_fraction(amax, fmax):
    a = Fraction(amax)
    f = Fraction(fmax)
    e = -200
    while a > f * Fraction(2) ** e:
        e += 1
    return e


def test_shared_exponent_closed_forms():
    se = F.shared_exponent
    assert se(448.0, 448.0) == 0
    assert se(np.nextafter(448.0, 1e9), 448.0) == 1
    assert se(224.0, 448.0) == -1
    assert se(6.0, 6.0) == 0
    assert se(6.0 * 2 ** -5, 6.0) == -5
    assert se(np.nextafter(6.0, 10), 6.0) == 1
    assert se(1.0, 6.0) == -2            # 6/4 >= 1 > 6/8
    assert se(0.0, 6.0) == -127
    assert se(1e300, 448.0) == 127       # clamped
    assert se(1e-300, 6.0) == -127       # clamped


def test_shared_exponent_brute_force():
    rng = np.random.default_rng(0)
    a = np.ldexp(rng.uniform(0.5, 1.0, 2000), rng.integers(-60, 60, 2000))
    edge = np.ldexp(np.array([448.0, 6.0, 7.0, 3.0]), 3)
    a = np.concatenate([a, edge, np.nextafter(edge, 0), np.nextafter(edge, np.inf)])
    for fmax in (448.0, 6.0):
        got = F.shared_exponent(a, fmax)
        ref = np.array([_smallest_exponent_fraction(x, fmax) for x in a])
        assert np.array_equal(got, np.clip(ref, -127, 127))


def test_fp8_block_quant_uses_whole_block_scale():
    rng = np.random.default_rng(1)
    t = rng.normal(size=(3, 16, 8))
    codes, e = Q.quantize_fp8_block(t)
    for b in range(3):
        amax = np.abs(t[b]).max()
        assert amax <= 448 * 2.0 ** e[b] and amax > 448 * 2.0 ** (e[b] - 1)
    deq = Q.dequant_fp8_block(codes, e)
    # relative error of E4M3 normals is at most 2^-4
    big = np.abs(t) > 2.0 ** (e[:, None, None] - 6 + 0)
    assert np.all(np.abs(deq - t)[big] <= 2.0 ** -4 * np.abs(t)[big] + 1e-300)


def test_mx_groups_run_along_last_axis():
    # values constant within each 32-group but spanning 2^0..2^7 across groups: exact
    x = np.repeat(2.0 ** np.arange(8), 32)[None, :] * np.array([[1.0], [-1.0]])
    codes, e = Q.quantize_mx_lastaxis(x)
    assert e.shape == (2, 8)
    assert np.array_equal(Q.dequant_mx_lastaxis(codes, e), x)
    # a group holding 1 and 64 loses the 1 (scale 2^4, 1/16 -> 0)
    y = np.zeros((1, 32))
    y[0, 0], y[0, 1] = 64.0, 1.0
    c, e = Q.quantize_mx_lastaxis(y)
    assert e[0, 0] == 4 and Q.dequant_mx_lastaxis(c, e)[0, 1] == 0.0


def test_operand_groups_q_along_d_v_along_slots():
    # q, k constant along d per token; v constant along slots per channel:
    # with groups along the right axes every MXFP4 group is constant -> exact
    bs, d = 32, 64
    q = np.tile(2.0 ** (np.arange(bs) % 8)[:, None], (1, d))[None]
    v = np.tile((2.0 ** (np.arange(d) % 8) * (-1.0) ** np.arange(d))[None, :], (bs, 1))[None]
    ops = Q.prepare_operands(q, q, v)
    assert np.array_equal(ops["q4_deq"], q)
    assert np.array_equal(ops["k4_deq"], q)
    assert np.array_equal(ops["v4_deq"], v)
    assert ops["v4t"].shape == (1, d, bs) and ops["v4t_exp"].shape == (1, d, 1)
    assert ops["q4_exp"].shape == (1, bs, d // 32)
