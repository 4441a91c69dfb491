"""The page orders the C header documents (restated in gpu_support and used
by the GPU tests to read device pages): each is a permutation of the page,
and where the reordered form applies, the 16 bytes lane l of a 64-lane load
holds are bytes 16l .. 16l + 15 of a 1 KB run, already in operand order."""

import numpy as np
import pytest

from gpu_support import k16_index, k8_index, v8_index


@pytest.mark.parametrize("bs,d", [(16, 64), (16, 128), (32, 64), (32, 128), (16, 32), (48, 96),
                                  (8, 128), (16, 48), (1, 64), (128, 128)])
def test_bf16_k_order_is_a_permutation(bs, d):
    idx = k16_index(bs, d)
    assert sorted(idx.ravel().tolist()) == list(range(bs * d))
    if bs % 16 or d % 32:
        np.testing.assert_array_equal(idx, np.arange(bs * d).reshape(bs, d))


@pytest.mark.parametrize("bs,d", [(16, 64), (16, 128), (32, 128), (16, 256)])
def test_bf16_k_lane_runs(bs, d):
    # Lane l = 16 grp + n of load j in tile tt holds token 16 tt + n, values
    # d = 32 j + 8 grp .. +7: elements (64 j + l) * 8 .. +7 of the tile.
    idx = k16_index(bs, d)
    for tt in range(bs // 16):
        for j in range(d // 32):
            for lane in range(64):
                n, grp = lane % 16, lane // 16
                got = idx[16 * tt + n, 32 * j + 8 * grp:32 * j + 8 * grp + 8]
                base = tt * 16 * d + (64 * j + lane) * 8
                np.testing.assert_array_equal(got, np.arange(base, base + 8))


@pytest.mark.parametrize("bs,d", [(16, 64), (16, 128), (32, 64), (32, 128), (16, 256), (16, 32), (32, 16),
                                  (16, 48), (16, 192)])
def test_8bit_orders_are_permutations(bs, d):
    for idx in (k8_index(bs, d), v8_index(bs, d)):
        assert sorted(idx.ravel().tolist()) == list(range(bs * d))
    if d % 64:
        np.testing.assert_array_equal(k8_index(bs, d), np.arange(bs * d).reshape(bs, d))


@pytest.mark.parametrize("bs,d", [(16, 64), (16, 128), (32, 128), (16, 256)])
def test_8bit_lane_runs(bs, d):
    # K: lane l = 16 grp + n, load w of tile tt holds token 16 tt + n, codes
    # d = grp * d/4 + 16 w .. +15.  V: lane l = row r holds codes of d =
    # 16 * (c // 4) + n ... for byte c = 16 w .. 16 w + 15 of the row.
    k, v = k8_index(bs, d), v8_index(bs, d)
    span = d // 4
    for tt in range(bs // 16):
        for w in range(span // 16):
            for lane in range(64):
                n, grp = lane % 16, lane // 16
                base = tt * 16 * d + (64 * w + lane) * 16
                got = k[16 * tt + n, grp * span + 16 * w:grp * span + 16 * w + 16]
                np.testing.assert_array_equal(got, np.arange(base, base + 16))
                # V row r = lane: tokens 16 tt + 4 (r // 16) + (c % 4), d = 16 (c // 4) + r % 16
                vb = [v[16 * tt + 4 * (lane // 16) + c % 4, 16 * (c // 4) + lane % 16]
                      for c in range(16 * w, 16 * w + 16)]
                assert vb == list(range(base, base + 16))
