"""Per-row absmax quantisation of K/V rows to 8-bit floating-point codes.

Test infrastructure only (see the package docstring).

This is the per-row absmax scheme of the vladkulikov.com notebook "Модуль 10.
KV-кэши и эффективный инференс" (the KV-compression experiment; see
:mod:`oracle.quant`) with the integer code replaced by an 8-bit float.  The
pages fix only the integer codes; the 8-bit float variant and its format are
readings taken here:

* the format is E4M3 with no infinities: bit 7 sign, bits 6..3 a biased
  exponent (bias 7), bits 2..0 the mantissa.  Exponent field 0 holds the
  subnormals ``m * 2**-9``; otherwise the value is ``(1 + m / 8) *
  2**(e - 7)``.  The all-ones magnitude ``0x7F`` is not a number and is
  never produced; the largest finite magnitude is ``0x7E = 448``;
* the row's scale is its largest magnitude divided by 448 (all-zero row:
  scale 1), decided in float64 as for the integer codes;
* each value ``x / scale`` (float64) goes to the nearest representable
  value, ties to the even code (mantissa bit 0 clear), magnitudes above 448
  to 448; a zero (of either sign) gets code 0x00;
* the stored scale is the nearest fp32 of the float64 scale, and the value
  read back is ``decode(code) * fp32(scale)``.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL_EXP = -6  # smallest exponent of a normal value
_MANT_BITS = 3


def e4m3_decode(codes):
    """Values of 8-bit codes (uint8 array) as float64; NaN for 0x7F / 0xFF."""
    c = np.asarray(codes, dtype=np.int64)
    if np.any((c < 0) | (c > 255)):
        raise ValueError("codes must be bytes")
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = m * 2.0 ** -9
    out = sign * np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def e4m3_round(y):
    """Nearest E4M3 value of each float64 in ``y`` (ties to the even code,
    magnitudes beyond 448 to 448), as float64."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), E4M3_MAX)
    _, k = np.frexp(a)  # a = f * 2**k, f in [0.5, 1): floor(log2 a) = k - 1
    e = np.maximum(k - 1, _MIN_NORMAL_EXP)
    quantum = np.exp2((e - _MANT_BITS).astype(np.float64))
    r = np.rint(a / quantum) * quantum  # the division by a power of two is exact
    r = np.where(a == 0, 0.0, r)
    return np.copysign(r, y)


def e4m3_encode(values):
    """Codes (uint8) of values that are E4M3 values (``e4m3_round`` output)."""
    v = np.asarray(values, dtype=np.float64)
    a = np.abs(v)
    if np.any(a > E4M3_MAX) or np.any(np.isnan(v)):
        raise ValueError("values must be finite E4M3 values")
    sign = np.where(v < 0, 0x80, 0)
    _, k = np.frexp(a)
    e_unb = k - 1
    sub = a < 2.0 ** _MIN_NORMAL_EXP
    m_sub = a / 2.0 ** -9
    m_norm = a / np.exp2((e_unb - _MANT_BITS).astype(np.float64)) - 8.0
    m = np.where(sub, m_sub, m_norm)
    e = np.where(sub, 0, e_unb + 7)
    if np.any(m != np.rint(m)) or np.any((m < 0) | (m > 7)):
        raise ValueError("values must be E4M3 values")
    return (sign | (e.astype(np.int64) << 3) | m.astype(np.int64)).astype(np.uint8)


def quantize_rows_fp8(x):
    """Codes (uint8) and float64 scales of every row (last axis) of ``x``."""
    x = np.asarray(x, dtype=np.float64)
    scale = np.max(np.abs(x), axis=-1, keepdims=True) / E4M3_MAX
    scale = np.where(scale == 0, 1.0, scale)
    return e4m3_encode(e4m3_round(x / scale)), scale


def dequantize_rows_fp8(codes, scale):
    """Values read back from codes and (stored) scales."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)


def fake_quantize_rows_fp8(x):
    """Round trip through the stored form: code, fp32 scale, read back."""
    codes, scale = quantize_rows_fp8(x)
    stored = np.asarray(scale, dtype=np.float64).astype(np.float32).astype(np.float64)
    return dequantize_rows_fp8(codes, stored)
