"""Per-row absmax quantisation of K/V rows, as the oracle defines it.

Test infrastructure only (see the package docstring).

Source: vladkulikov.com notebook "Модуль 10. KV-кэши и эффективный инференс",
the KV-compression experiment (``fake_quantize_rows`` and the byte count of
"ideal packed codes + scales" that follows it).  A row is one token's
``head_dim`` values for one KV head.  With ``limit = 2**(bits - 1) - 1``:

* the row's scale is its largest magnitude divided by ``limit``; an all-zero
  row gets scale 1;
* each code is ``x / scale`` rounded to the nearest integer, ties to even
  (numpy ``rint``), then clipped to ``[-limit, limit]``;
* the value read back is ``code * scale``.

The notebook keeps the scale in float64 for its experiment and counts four
bytes (fp32) per row and per K/V for the packed layout.  Readings taken here:

* the code is decided in float64 (the notebook's precision): the scale is
  ``absmax / limit`` in float64 and the code is ``rint(x / scale)`` in
  float64;
* the stored scale is that float64 scale rounded to the nearest fp32, and
  the value read back is ``code * fp32(scale)`` (the packed form has only
  the fp32 scale).
"""

from __future__ import annotations

import numpy as np


def code_limit(bits):
    """Largest code magnitude for a signed ``bits``-bit code (symmetric range)."""
    if isinstance(bits, bool) or not isinstance(bits, (int, np.integer)) or not 2 <= bits <= 8:
        raise ValueError("bits must be an integer in 2..8")
    return 2 ** (int(bits) - 1) - 1


def quantize_rows(x, bits=8):
    """Codes and float64 scales of every row (last axis) of ``x``.

    Returns ``(codes, scale)``: ``codes`` int64 with ``x``'s shape, ``scale``
    float64 with the last axis kept as length 1.
    """
    x = np.asarray(x, dtype=np.float64)
    limit = code_limit(bits)
    scale = np.max(np.abs(x), axis=-1, keepdims=True) / limit
    scale = np.where(scale == 0, 1.0, scale)
    codes = np.clip(np.rint(x / scale), -limit, limit).astype(np.int64)
    return codes, scale


def stored_scale(scale):
    """The scale as the packed layout keeps it: nearest fp32, held in float64."""
    return np.asarray(scale, dtype=np.float64).astype(np.float32).astype(np.float64)


def dequantize_rows(codes, scale):
    """Values read back from codes and (stored) scales."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scale, dtype=np.float64)


def fake_quantize_rows(x, bits=8):
    """Round trip through the packed form: code, fp32 scale, read back."""
    codes, scale = quantize_rows(x, bits)
    return dequantize_rows(codes, stored_scale(scale))


def packed_bytes(n_tokens, head_dim, bits=8):
    """Bytes of ideally packed K and V codes plus one fp32 scale per row of
    each, for ``n_tokens`` rows of ``head_dim`` values (one KV head)."""
    code_limit(bits)
    return 2 * n_tokens * head_dim * bits / 8 + 2 * n_tokens * 4
