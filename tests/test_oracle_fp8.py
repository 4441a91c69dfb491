"""Pins of the oracle's 8-bit float (E4M3, no infinities) row quantisation.

The format is a reading (the pages fix only integer codes); these tests pin
the oracle to the format's definition through independent routes: the value
table rebuilt through IEEE half precision (every E4M3 value is a half), a
brute-force nearest-value search with the tie rule, and the row scheme's
invariants (the row maximum maps to +-448, zero rows, scale invariance).
"""

import numpy as np
import pytest

from oracle.fp8 import (E4M3_MAX, dequantize_rows_fp8, e4m3_decode, e4m3_encode, e4m3_round,
                        fake_quantize_rows_fp8, quantize_rows_fp8)


def _via_half(code):
    """E4M3 code -> value through float16 bits (exponent rebiased 7 -> 15,
    mantissa shifted to the top of the half's 10 bits)."""
    s, e, m = code >> 7, (code >> 3) & 0xF, code & 7
    if e == 0:
        if m == 0:
            return 0.0
        # subnormal m * 2**-9 = normal half with exponent of the leading bit
        lead = m.bit_length() - 1
        frac = (m - (1 << lead)) << (10 - lead)
        bits = (s << 15) | ((lead - 9 + 15) << 10) | frac
    else:
        bits = (s << 15) | ((e - 7 + 15) << 10) | (m << 7)
    return float(np.array([bits], dtype=np.uint16).view(np.float16)[0])


def _finite_codes():
    return np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def test_decode_table_matches_half_precision_route():
    for c in range(256):
        v = e4m3_decode(np.uint8(c))
        if (c & 0x7F) == 0x7F:
            assert np.isnan(v)
        else:
            assert v == _via_half(c), c


def test_decode_landmarks():
    assert e4m3_decode(np.uint8(0x00)) == 0.0
    assert e4m3_decode(np.uint8(0x01)) == 2.0 ** -9
    assert e4m3_decode(np.uint8(0x07)) == 7 * 2.0 ** -9
    assert e4m3_decode(np.uint8(0x08)) == 2.0 ** -6
    assert e4m3_decode(np.uint8(0x38)) == 1.0
    assert e4m3_decode(np.uint8(0x7E)) == E4M3_MAX == 448.0
    assert e4m3_decode(np.uint8(0xB8)) == -1.0
    pos = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)  # codes 0..0x7E ascend
    assert len(set(e4m3_decode(_finite_codes()).tolist())) == 253  # +0 and -0 coincide


def test_encode_inverts_decode():
    codes = _finite_codes()
    vals = e4m3_decode(codes)
    back = e4m3_encode(vals)
    want = np.where(codes == 0x80, 0x00, codes)  # -0 is written as code 0
    np.testing.assert_array_equal(back, want)


def _brute_round(y, table, table_codes):
    a = min(abs(y), E4M3_MAX)
    d = np.abs(table - a)
    best = np.flatnonzero(d == d.min())
    if len(best) > 1:  # a tie: the even code
        best = [b for b in best if table_codes[b] % 2 == 0]
    return float(np.copysign(table[best[0]], y))


def test_round_is_nearest_with_even_ties_brute_force():
    codes = np.arange(0x7F, dtype=np.uint8)
    table = e4m3_decode(codes)
    rng = np.random.default_rng(0)
    ys = np.concatenate([rng.normal(size=400) * 10.0 ** rng.integers(-4, 3, size=400),
                         rng.uniform(-460, 460, size=200)])
    # exact midpoints between neighbours, and their close neighbours
    mids = (table[1:] + table[:-1]) / 2
    ys = np.concatenate([ys, mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9)])
    got = e4m3_round(ys)
    for y, g in zip(ys, got):
        assert g == _brute_round(y, table, codes), y


def test_round_keeps_representable_values_and_saturates():
    vals = e4m3_decode(_finite_codes())
    np.testing.assert_array_equal(e4m3_round(vals), vals)
    np.testing.assert_array_equal(e4m3_round(np.array([448.0, 460.0, 1e6, -1e6])), [448, 448, 448, -448])


def test_row_scheme_invariants():
    rng = np.random.default_rng(1)
    x = rng.normal(size=(50, 128))
    codes, scale = quantize_rows_fp8(x)
    # the row's largest magnitude maps to +-448 exactly
    idx = np.argmax(np.abs(x), axis=-1)
    top = codes[np.arange(50), idx]
    assert np.all((top & 0x7F) == 0x7E)
    assert np.all((top >> 7) == (x[np.arange(50), idx] < 0))
    np.testing.assert_allclose(scale[:, 0], np.abs(x).max(-1) / 448)
    # scale invariance by powers of two and sign symmetry
    c2, s2 = quantize_rows_fp8(x * 8.0)
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(s2, scale * 8.0)
    cn, _ = quantize_rows_fp8(-x)
    np.testing.assert_array_equal(cn, codes ^ 0x80)
    # zero rows: scale 1, codes 0
    cz, sz = quantize_rows_fp8(np.zeros((2, 16)))
    assert np.all(cz == 0) and np.all(sz == 1.0)
    # read-back error within half a quantum of each value (3 mantissa bits: <= 2**-4 relative
    # for normals) plus the fp32 rounding of the scale
    back = fake_quantize_rows_fp8(x)
    rel = np.abs(back - x) / np.maximum(np.abs(x), scale * 2.0 ** -6)
    assert rel.max() <= 2.0 ** -4 * (1 + 1e-6)
    np.testing.assert_array_equal(dequantize_rows_fp8(codes, scale), e4m3_decode(codes) * scale)


def test_encode_rejects_non_representable():
    with pytest.raises(ValueError):
        e4m3_encode(np.array([0.3]))
    with pytest.raises(ValueError):
        e4m3_encode(np.array([449.0]))


def test_pool_stores_fp8_codes_and_reads_back():
    """A Pool(quant_fp8=True) keeps the codes and fp32 scales of each row and
    attends over the values they read back; copy-on-write copies them."""
    import oracle
    rng = np.random.default_rng(3)
    p = oracle.Pool(6, 4, 2, 16, quant_fp8=True)
    p.create(0)
    k, v = rng.normal(size=(5, 2, 16)), rng.normal(size=(5, 2, 16))
    slots = p.append(0, 5)
    p.write(slots, k, v)
    for i, slot in enumerate(slots):
        b, o = divmod(slot, 4)
        codes, scale = quantize_rows_fp8(k[i])
        np.testing.assert_array_equal(p.Kc[b, o], codes)
        np.testing.assert_array_equal(p.Ks[b, o], scale[:, 0].astype(np.float32).astype(np.float64))
        np.testing.assert_array_equal(p.K[b, o], fake_quantize_rows_fp8(k[i]))
    p.share(0, 1, 5)
    s2 = p.append(1, 1)  # copy-on-write of the shared partial block
    b_new, b_old = divmod(s2[0], 4)[0], p.tables[0][-1]
    np.testing.assert_array_equal(p.Kc[b_new, :1], p.Kc[b_old, :1])
    with pytest.raises(ValueError):
        oracle.Pool(4, 4, 1, 4, quant_bits=4, quant_fp8=True)
