"""The gfx950 behaviour the kernels are built on, measured on the GPU through
libda2_probes.so (MI355X only). These are design assumptions, not parity
checks: if one of them fails, the kernel that relies on it is wrong.

* v_cvt_scalef32_pk_bf16_fp8 (scale 1) widens every finite E4M3 code exactly,
  from any byte position: the fp8 tiles' QK^T feeds bf16 MFMAs with it.
* v_cvt_pk_fp8_f32 rounds to nearest even over the E4M3 range: the P codes of
  fp8 tiles and the operand codes are computed with it.
* v_cvt_scalef32_pk_fp4_f32 (scale 1) rounds to nearest even over the E2M1
  range and saturates at 6.
* v_cvt_scalef32_pk_fp8_bf16 and v_cvt_scalef32_pk_fp4_bf16 give the codes
  of x / scale, rounded to nearest even, for every bf16 value x and the
  power-of-two scales the preparation kernel passes (2^-100 and up): it
  converts the operands with them, straight from the packed bf16 words.
* bf16 MFMAs over exactly widened E4M3 values give the fp32 sum of exact
  products, while one scaled f8f6f4 MFMA over the same codes does not: it
  keeps only a limited number of bits below the largest product. Neither do
  the unscaled 32x32x16 fp8 MFMAs, which also issue at the bf16 rate. This is
  why the fp8 tiles' QK^T, whose rounding decides P codes, runs on bf16 MFMAs.
"""

import numpy as np
import pytest
import torch

from oracle import formats as F

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def probes():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_sparse_mixed_amd import probes as P
    return P


def _e4m3_values():
    codes = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    return codes, vals


def test_widening_e4m3_to_bf16_is_exact(probes):
    got = probes.widen_fp8()                                   # [256][4] bf16 bits
    codes, vals = _e4m3_values()
    want = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    finite = np.isfinite(vals)
    assert finite.sum() == 254
    for p in range(4):
        assert np.array_equal(got[finite, p], want[finite]), f"byte position {p}"


def test_fp32_to_e4m3_rounds_to_nearest_even(probes):
    codes, vals = _e4m3_values()
    v = np.sort(np.unique(vals[np.isfinite(vals) & (vals >= 0)]))
    mids = (v[:-1] + v[1:]) / 2                                 # every tie
    rng = np.random.default_rng(0)
    rand = rng.uniform(-448, 448, 20000) * rng.choice([1, 1e-2, 1e-4], 20000)
    x = np.concatenate([v, -v, mids, -mids, rand]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    got = probes.to_fp8(x)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)
    assert np.array_equal(got, F.encode_e4m3(x.astype(np.float64)))


def test_fp32_to_e2m1_rounds_to_nearest_even_and_saturates(probes):
    v = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    mids = (v[:-1] + v[1:]) / 2
    rng = np.random.default_rng(1)
    inside = np.concatenate([v, -v, mids, -mids, rng.uniform(-6, 6, 5000)]).astype(np.float32)
    got = probes.to_fp4(inside)
    assert np.array_equal(got, F.encode_e2m1(inside.astype(np.float64)))
    above = np.array([6.5, 7.0, 100.0, -6.5, -1e6], dtype=np.float32)
    assert np.array_equal(probes.to_fp4(above), np.array([7, 7, 7, 15, 15], dtype=np.uint8))


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
def test_bf16_scaled_conversion_divides_by_the_scale(probes, fmt):
    lim, enc = (448.0, F.encode_e4m3) if fmt == "fp8" else (6.0, F.encode_e2m1)
    bits = np.arange(1 << 16, dtype=np.uint32)
    vals = (bits << 16).view(np.float32).astype(np.float64)
    finite = np.isfinite(vals)
    for e in (-100, -20, -3, 0, 3, 20, 100):
        sc = 2.0 ** e
        y = np.where(finite, vals, 0.0) / sc
        keep = finite & (np.abs(y) <= lim)
        xb = bits[keep].astype(np.uint16)
        if xb.size % 2:
            xb = xb[:-1]
        got = probes.bf16_to(xb, sc, fmt)
        want = enc((xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64) / sc)
        assert np.array_equal(got, want), f"{fmt} scale 2^{e}: {int((got != want).sum())} of {xb.size} codes differ"


def _outlier_codes(rng, scale_idx):
    """E4M3 code matrices [32][64] of N(0,1)-like values, with two outlier
    channels (k indices) scaled x8, like the Small workload."""
    x = rng.standard_normal((32, 64))
    x[:, scale_idx] *= 8
    x = x / np.abs(x).max() * 400
    return F.encode_e4m3(x)


def test_bf16_mfma_is_exact_and_the_f8f6f4_mfma_is_not(probes):
    # a case with one large product: exact sum 448 * 448 + 63 * 1 = 200767,
    # representable in fp32
    one, big = 0x38, 0x7E
    a = np.full((32, 64), one, dtype=np.uint8)
    b = np.full((32, 64), one, dtype=np.uint8)
    a[:, 0] = big
    b[:, 0] = big
    exact = 448.0 * 448.0 + 63.0
    d16 = probes.mfma_fp8(a, b, path="bf16")
    d8 = probes.mfma_fp8(a, b, path="f8f6f4")
    d8k16 = probes.mfma_fp8(a, b, path="fp8_k16")
    assert np.all(d16 == exact)
    assert np.all(d8 != exact)
    assert np.all(d8k16 != exact)
    # random operands with outlier channels: bf16 path within fp32 rounding of
    # the exact sum; the f8f6f4 path's error relative to the largest product
    rng = np.random.default_rng(2)
    worst16 = worst8 = worst8k16 = 0.0
    for t in range(8):
        idx = rng.choice(64, 2, replace=False)
        a, b = _outlier_codes(rng, idx), _outlier_codes(rng, idx)
        av, bv = F.decode_e4m3(a), F.decode_e4m3(b)
        ex = av @ bv.T
        big_prod = np.abs(av[:, None, :] * bv[None, :, :]).max(axis=2)
        absum = np.abs(av) @ np.abs(bv).T
        d16 = probes.mfma_fp8(a, b, path="bf16")
        d8 = probes.mfma_fp8(a, b, path="f8f6f4")
        d8k16 = probes.mfma_fp8(a, b, path="fp8_k16")
        worst16 = max(worst16, float((np.abs(d16 - ex) / absum).max()))
        worst8 = max(worst8, float((np.abs(d8 - ex) / big_prod).max()))
        worst8k16 = max(worst8k16, float((np.abs(d8k16 - ex) / big_prod).max()))
    print(f"[gpu] bf16 path: max |err| / sum|products| = {worst16:.2e}; "
          f"f8f6f4 path: max |err| / largest product = {worst8:.2e} (2^{np.log2(max(worst8, 1e-300)):.1f}); "
          f"fp8 32x32x16 path: {worst8k16:.2e} (2^{np.log2(max(worst8k16, 1e-300)):.1f})")
    assert worst16 <= 64 * 2.0 ** -24
    assert worst8 > 64 * 2.0 ** -24
    assert worst8k16 > 64 * 2.0 ** -24


@pytest.mark.gpu
def test_f64_mfma_result_rows_are_lane_group_plus_four_element(probes):
    # The layout the draft logits kernel builds on: lane l feeds A[l % 16][l / 16]
    # and B[l / 16][l % 16], and its result element e is D[l / 16 + 4 e][l % 16].
    # With distinct small integers the product is exact, so any other row map
    # shows as a mismatch.
    rng = np.random.default_rng(3)
    a = rng.integers(-8, 9, size=(16, 4)).astype(np.float64)
    b = rng.integers(-8, 9, size=(4, 16)).astype(np.float64)
    a[:, 0] += 100.0 * np.arange(16)        # every row of A @ B distinct
    d = probes.mfma_f64(a, b)
    assert np.array_equal(d, a @ b)
