"""Pins of the oracle's per-row absmax quantisation (oracle.quant) and of a
quantised oracle pool.

Source: vladkulikov.com notebook "Модуль 10. KV-кэши и эффективный
инференс", KV-compression experiment.

* The notebook's own checks: an all-zero 2 x 4 block quantises to zeros at
  3 bits; with 8-bit codes the attention output of random normal keys,
  values and queries (128 tokens, head_dim 32, 12 queries) stays within 3%
  relative (Frobenius) error of the float64 output; the packed size of codes
  plus fp32 scales is 2 n d bits / 8 + 2 n 4 bytes.
* Worked rows whose scale is exact in binary (absmax = limit * 2^k), so the
  codes are known by hand, including ties that must round to even.
* Properties for random rows: |x - read back| <= scale / 2 (plus the fp32
  scale rounding), the largest code magnitude of a non-zero row is the
  limit, codes carry the sign of x, zero rows read back exactly.
* A quantised pool stores exactly those codes and scales and copies them on
  copy-on-write.
* Planted mistakes (half-away-from-zero rounding, no zero-row guard, an
  unsigned limit 2^bits - 1) each fail a pin.
"""

import numpy as np
import pytest

from oracle import (Pool, attention, code_limit, dequantize_rows, fake_quantize_rows,
                    packed_bytes, quantize_rows, stored_scale)


def test_zero_rows_read_back_zero():
    # The notebook's assertion on a 2 x 4 zero block at 3 bits.
    np.testing.assert_array_equal(fake_quantize_rows(np.zeros((2, 4)), 3), 0)
    codes, scale = quantize_rows(np.zeros((3, 8)), 8)
    assert (codes == 0).all() and (scale == 1.0).all()


def test_limits():
    assert code_limit(8) == 127 and code_limit(3) == 3 and code_limit(4) == 7
    for bad in (1, 9, 8.0, True):
        with pytest.raises(ValueError):
            code_limit(bad)


def test_worked_rows_ties_to_even():
    # absmax 127 -> scale exactly 1: codes are rint(x), ties to even.
    row = np.array([[127.0, -63.5, 31.75, 0.5, -0.5, 1.5, 2.5, -2.5]])
    codes, scale = quantize_rows(row, 8)
    assert scale[0, 0] == 1.0
    assert codes[0].tolist() == [127, -64, 32, 0, 0, 2, 2, -2]
    # absmax 15.875 = 127 / 8 -> scale 0.125: x / scale = [127, -8, 0.5, 1.5]
    row = np.array([[15.875, -1.0, 0.0625, 0.1875]])
    codes, scale = quantize_rows(row, 8)
    assert scale[0, 0] == 0.125
    assert codes[0].tolist() == [127, -8, 0, 2]
    np.testing.assert_array_equal(fake_quantize_rows(row, 8), [[15.875, -1.0, 0.0, 0.25]])
    # 3 bits: limit 3, absmax 3 -> scale 1.
    codes, _ = quantize_rows(np.array([[3.0, 1.5, -2.5, 0.4, -3.0]]), 3)
    assert codes[0].tolist() == [3, 2, -2, 0, -3]


def test_random_rows_error_bound_and_extremes():
    rng = np.random.default_rng(31)
    x = rng.standard_normal((64, 128)) * rng.uniform(0.01, 10.0, size=(64, 1))
    x[5] = 0.0
    codes, scale = quantize_rows(x, 8)
    s32 = stored_scale(scale)
    back = dequantize_rows(codes, s32)
    bound = scale / 2 + 127 * np.abs(s32 - scale) + 1e-12 * scale
    assert (np.abs(x - back) <= bound).all()
    assert (np.abs(codes) <= 127).all()
    nonzero = np.abs(x).max(axis=1) > 0
    assert (np.abs(codes[nonzero]).max(axis=1) == 127).all()
    assert (np.sign(codes) * np.sign(x) >= 0).all()
    np.testing.assert_array_equal(back[5], 0.0)
    # The stored scale is the nearest fp32 of absmax / 127.
    np.testing.assert_array_equal(s32, np.float32(scale).astype(np.float64))


def test_notebook_experiment_error_and_bytes():
    rng = np.random.default_rng(1010)
    n, d = 128, 32
    keys = rng.normal(size=(n, d))
    values = rng.normal(size=(n, d))
    queries = rng.normal(size=(12, d))
    errors = {}
    for bits in (8, 3):
        kq, vq = fake_quantize_rows(keys, bits), fake_quantize_rows(values, bits)
        # 12 queries against all 128 keys: 12 decode rows of one head.
        out = np.concatenate([attention(queries[i:i + 1, None, :], kq[:, None, :], vq[:, None, :])
                              for i in range(12)])
        full = np.concatenate([attention(queries[i:i + 1, None, :], keys[:, None, :], values[:, None, :])
                               for i in range(12)])
        errors[bits] = np.linalg.norm(out - full) / np.linalg.norm(full)
    assert errors[8] < 0.03
    assert errors[3] > errors[8]
    assert packed_bytes(n, d, 8) == 2 * n * d + 2 * n * 4 == 9216
    assert packed_bytes(n, d, 3) == 4096


def test_quantised_pool_stores_codes_and_copies_them():
    rng = np.random.default_rng(7)
    pool = Pool(8, 4, num_kv_heads=2, head_dim=16, quant_bits=8)
    pool.create("a")
    slots = pool.append("a", 6)
    k = rng.standard_normal((6, 2, 16))
    v = rng.standard_normal((6, 2, 16))
    k[2, 1] = 0.0
    pool.write(slots, k, v)
    keys, values = pool.gather("a")
    np.testing.assert_array_equal(keys, fake_quantize_rows(k, 8))
    np.testing.assert_array_equal(values, fake_quantize_rows(v, 8))
    codes, scale = quantize_rows(k, 8)
    for i, slot in enumerate(slots):
        blk, off = divmod(slot, 4)
        np.testing.assert_array_equal(pool.Kc[blk, off], codes[i])
        np.testing.assert_array_equal(pool.Ks[blk, off], stored_scale(scale[i, :, 0]))
    # fork + append into the shared partial tail: the copy carries codes and scales.
    pool.fork("a", "b")
    pool.append("b", 1)
    old, new = pool.copies[-1]
    for arr in (pool.Kc, pool.Vc, pool.Ks, pool.Vs, pool.K, pool.V):
        np.testing.assert_array_equal(arr[new], arr[old])


# ------------------------------------------------------------ planted mistakes
def _mutant_half_away(x, bits):
    x = np.asarray(x, dtype=np.float64)
    limit = code_limit(bits)
    scale = np.max(np.abs(x), axis=-1, keepdims=True) / limit
    scale = np.where(scale == 0, 1.0, scale)
    codes = np.clip(np.sign(x / scale) * np.floor(np.abs(x / scale) + 0.5), -limit, limit)
    return codes, scale


def _mutant_no_zero_guard(x, bits):
    x = np.asarray(x, dtype=np.float64)
    limit = code_limit(bits)
    scale = np.max(np.abs(x), axis=-1, keepdims=True) / limit
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.clip(np.rint(x / scale), -limit, limit), scale


def _mutant_unsigned_limit(x, bits):
    x = np.asarray(x, dtype=np.float64)
    limit = 2 ** bits - 1
    scale = np.max(np.abs(x), axis=-1, keepdims=True) / limit
    scale = np.where(scale == 0, 1.0, scale)
    return np.clip(np.rint(x / scale), -limit, limit), scale


def test_pins_reject_planted_mistakes():
    row = np.array([[127.0, -63.5, 31.75, 0.5, -0.5, 1.5, 2.5, -2.5]])
    assert _mutant_half_away(row, 8)[0][0].tolist() != [127, -64, 32, 0, 0, 2, 2, -2]
    codes, scale = _mutant_no_zero_guard(np.zeros((2, 4)), 3)
    assert not np.array_equal(codes * scale, np.zeros((2, 4)))
    codes, _ = _mutant_unsigned_limit(row, 8)
    assert np.abs(codes).max() != 127
