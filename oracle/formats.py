"""Number formats, decoded from their definitions and encoded by nearest search.

[OFP8] E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits. Exponent field 0
holds subnormals m/8 * 2^-6; the all-ones exponent with all-ones mantissa is
NaN; there are no infinities; the largest finite magnitude is 448.

[OCP-MX] FP4 E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent
field 0 holds the subnormal 0.5; no infinities or NaN; magnitudes
{0, 0.5, 1, 1.5, 2, 3, 4, 6}. E8M0 scale code k stands for 2^(k - 127).

Encoding is round-to-nearest, ties to the even code (the code whose last
mantissa bit is 0), done by searching the decoded table. Inputs must lie
within the format's range; the callers guarantee it by their scale choice.
"""

from __future__ import annotations

import numpy as np


def _minifloat_value(code: int, ebits: int, mbits: int, bias: int) -> float:
    sign = -1.0 if (code >> (ebits + mbits)) & 1 else 1.0
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    if e == 0:
        return sign * (m / (1 << mbits)) * 2.0 ** (1 - bias)
    return sign * (1.0 + m / (1 << mbits)) * 2.0 ** (e - bias)


def _e4m3_table() -> np.ndarray:
    vals = np.array([_minifloat_value(c, 4, 3, 7) for c in range(256)])
    vals[0x7F] = np.nan
    vals[0xFF] = np.nan
    return vals


E4M3_VALUES = _e4m3_table()
E2M1_VALUES = np.array([_minifloat_value(c, 2, 1, 1) for c in range(16)])
E4M3_MAX = 448.0
E2M1_MAX = 6.0
E8M0_MIN_EXP = -127
E8M0_MAX_EXP = 127

# positive, finite codes in increasing order of value
_E4M3_POS = np.arange(0, 0x7F)      # 0x00 .. 0x7E
_E2M1_POS = np.arange(0, 8)


def decode_e4m3(codes) -> np.ndarray:
    return E4M3_VALUES[np.asarray(codes, dtype=np.int64)]


def decode_e2m1(codes) -> np.ndarray:
    return E2M1_VALUES[np.asarray(codes, dtype=np.int64)]


def _encode(values, table_vals: np.ndarray, sign_bit: int, fmax: float) -> np.ndarray:
    v = np.asarray(values, dtype=np.float64)
    mag = np.abs(v)
    if not np.all(mag <= fmax):
        raise ValueError("value outside the format's range")
    hi = np.searchsorted(table_vals, mag, side="left")          # table_vals[hi] >= mag
    hi = np.minimum(hi, len(table_vals) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - table_vals[lo]
    d_hi = table_vals[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(mag == table_vals[hi], hi, code)
    code = code | np.where(np.signbit(v), sign_bit, 0)
    return code.astype(np.uint8)


def encode_e4m3(values) -> np.ndarray:
    """Round to nearest E4M3 code, ties to even; |values| <= 448."""
    return _encode(values, E4M3_VALUES[_E4M3_POS], 0x80, E4M3_MAX)


def encode_e2m1(values) -> np.ndarray:
    """Round to nearest E2M1 code, ties to even; |values| <= 6."""
    return _encode(values, E2M1_VALUES[_E2M1_POS], 0x8, E2M1_MAX)


def shared_exponent(amax, fmax: float) -> np.ndarray:
    """Smallest integer e with amax <= fmax * 2^e, clamped to the E8M0 range.

    Reading: the pages fix no scale rule. This is the power-of-two scale that
    maps the group's largest magnitude into the format without clipping
    (unlike the OCP-MX informative rule floor(log2 amax) - emax, which can clip
    values between 6 and 8 times the scale). amax == 0 gives -127. The result
    is found by exact comparisons against ldexp(fmax, e); log2 is only used to
    pick a starting point.
    """
    a = np.asarray(amax, dtype=np.float64)
    out = np.full(a.shape, E8M0_MIN_EXP, dtype=np.int64)
    nz = a > 0
    if np.any(nz):
        an = a[nz]
        e = np.floor(np.log2(an)).astype(np.int64) - int(np.floor(np.log2(fmax))) - 1
        for _ in range(4):
            e = np.where(an > np.ldexp(fmax, e), e + 1, e)
        for _ in range(4):
            e = np.where(an <= np.ldexp(fmax, e - 1), e - 1, e)
        out[nz] = e
    return np.clip(out, E8M0_MIN_EXP, E8M0_MAX_EXP)
