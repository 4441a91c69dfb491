"""Pins of the oracle's attention against closed forms, brute force and
invariants the pages state.

* ferrum-kv 0.4.0 ``src/attention.rs`` unit tests: uniform attention over
  values 1, 2, 3 gives exactly 2; causal row 0 of a 3-row prefill is V0 and
  row 1 leans towards V1; a 4-token cache split over two 2-slot blocks
  averages into (10, 40).  The exact row values are worked out here from the
  softmax of two or three numbers.
* CMU 11-667 lecture 19 section 3: the tiled (online softmax) forward equals
  the two-pass one; ``online_softmax_stats`` gives (max, normaliser).
* The "Модуль 10" notebook: the chunked causal prefill covers exactly the
  query-key pairs of a one-shot prefill, so its outputs are equal.
* Invariants: GQA equals MHA with each KV head repeated; decode equals the
  last row of a causal prefill; a single visible key returns its value row;
  relabelling physical blocks changes nothing; paged gather equals the
  logical rows; shared prefixes with equal queries give equal outputs.
* Each planted mistake (a dropped scale, a top-left causal mask, interleaved
  instead of contiguous head groups) is shown to fail at least one pin.
"""

import math

import numpy as np
import pytest

from oracle import (Pool, attention, brute_force_attention, merge_partials,
                    combine_stats, online_softmax_stats, paged_attention, partial_attention,
                    tiled_attention)
from synth import logical_kv, append_stream, prefix_prefill, gqa_decode, tiny_fp32


def _pool_from_rows(keys, values, block_size, order=None, num_blocks=None):
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    n, hkv, d = keys.shape
    nb = num_blocks or max(1, -(-n // block_size))
    pool = Pool(nb, block_size, hkv, d, allocation_order=order)
    pool.create(0)
    slots = pool.append(0, n)
    pool.write(slots, keys, values)
    return pool


# ------------------------------------------------------------ ferrum-kv tests
def test_single_token_decode_uniform_is_two():
    heads, dim = 2, 4
    keys = np.ones((3, heads, dim))
    values = np.stack([np.full((heads, dim), pos + 1.0) for pos in range(3)])
    pool = _pool_from_rows(keys, values, 16, num_blocks=4)
    out = paged_attention(pool, 0, np.ones((1, heads, dim)))
    assert out.shape == (1, heads, dim)
    np.testing.assert_allclose(out, 2.0, rtol=0, atol=1e-14)


def _causal_case():
    rows = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    keys = rows[:, None, :]
    return keys, keys.copy(), keys.copy()


def test_prefill_causal_masking_closed_form():
    keys, values, q = _causal_case()
    pool = _pool_from_rows(keys, values, 16, num_blocks=2)
    out = paged_attention(pool, 0, q)[:, 0, :]
    # Row 0 sees only key 0: exactly V0.
    assert out[0].tolist() == [1.0, 0.0]
    # Row 1 sees scores [0, 1/sqrt 2]: weight of key 1 is a logistic.
    w1 = 1.0 / (1.0 + math.exp(-1.0 / math.sqrt(2.0)))
    np.testing.assert_allclose(out[1], [1.0 - w1, w1], rtol=0, atol=1e-15)
    assert out[1][0] < 0.5 < out[1][1]
    # Row 2 sees scores [1, 1, 2] / sqrt 2: weights 1 : 1 : e^(1/sqrt 2).
    e = math.exp(1.0 / math.sqrt(2.0))
    np.testing.assert_allclose(out[2], [(1 + e) / (2 + e)] * 2, rtol=0, atol=1e-15)
    np.testing.assert_allclose(out[1], [0.330238, 0.669762], atol=5e-7)
    np.testing.assert_allclose(out[2], [0.751745, 0.751745], atol=5e-7)


def test_attention_across_blocks_closed_form():
    dim = 2
    keys = np.stack([np.full((1, dim), pos + 1.0) for pos in range(4)])
    values = np.stack([np.full((1, dim), 10.0 * (pos + 1)) for pos in range(4)])
    pool = _pool_from_rows(keys, values, 2, order=[3, 1, 0, 2], num_blocks=4)
    assert pool.page_table(0) == (3, 1)
    out = paged_attention(pool, 0, np.ones((1, 1, dim)))[0, 0]
    w = np.exp(np.sqrt(2.0) * np.arange(1, 5))
    expected = 10.0 * (np.arange(1, 5) * w).sum() / w.sum()
    np.testing.assert_allclose(out, [expected, expected], rtol=0, atol=1e-12)
    assert 10.0 < out[0] < 40.0
    np.testing.assert_allclose(out[0], 36.928152, atol=5e-6)


# ------------------------------------------------------------ restatements
def _random_case(rng, q_len, kv_len, hq, hkv, d, scale=1.0):
    q = rng.standard_normal((q_len, hq, d)) * scale
    k = rng.standard_normal((kv_len, hkv, d)) * scale
    v = rng.standard_normal((kv_len, hkv, d))
    return q, k, v


@pytest.mark.parametrize("shape", [(1, 5, 2, 1, 3), (3, 7, 4, 2, 4), (4, 4, 6, 3, 2), (2, 9, 3, 3, 5)])
def test_brute_force_equals_vectorised(shape):
    rng = np.random.default_rng(sum(shape))
    q, k, v = _random_case(rng, *shape)
    np.testing.assert_allclose(attention(q, k, v), brute_force_attention(q, k, v), rtol=0, atol=1e-13)


@pytest.mark.parametrize("block", [1, 3, 16, 64])
def test_tiled_equals_two_pass(block):
    rng = np.random.default_rng(block)
    q, k, v = _random_case(rng, 9, 50, 8, 2, 16, scale=2.0)
    np.testing.assert_allclose(tiled_attention(q, k, v, block), attention(q, k, v), rtol=0, atol=1e-12)


def test_online_softmax_stats_is_max_and_normaliser():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(101) * 7
    blocks = [x[i:i + 13] for i in range(0, 101, 13)]
    m, l = online_softmax_stats(blocks)
    assert m == x.max()
    np.testing.assert_allclose(l, np.exp(x - x.max()).sum(), rtol=1e-14)


def test_online_stats_in_any_block_order_and_with_masked_blocks():
    """The fold does not depend on how the scores are cut into blocks or in
    which order the blocks come, and an empty or wholly masked block (all
    -inf) contributes nothing."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal(40) * 5
    want = (x.max(), np.exp(x - x.max()).sum())
    cuts = [x[:7], np.array([]), x[7:30], np.full(3, -np.inf), x[30:]]
    for blocks in (cuts, cuts[::-1], [x[i:i + 1] for i in range(40)]):
        m, l = online_softmax_stats(blocks)
        assert m == want[0]
        np.testing.assert_allclose(l, want[1], rtol=1e-13)
    assert online_softmax_stats([np.full(2, -np.inf)]) == (-np.inf, 0.0)
    assert combine_stats((1.5, 2.0), (-np.inf, 0.0)) == (1.5, 2.0)
    # Two equal maxima add their normalisers.
    assert combine_stats((0.0, 1.0), (0.0, 3.0)) == (0.0, 4.0)


def test_partials_merge_to_attention():
    rng = np.random.default_rng(7)
    q, k, v = _random_case(rng, 5, 37, 4, 2, 8, scale=3.0)
    edges = [0, 0, 6, 19, 19, 33, 37]      # includes empty ranges
    parts = [partial_attention(q, k, v, a, b) for a, b in zip(edges[:-1], edges[1:])]
    ms, ls, accs = zip(*parts)
    # Row 0 sees keys 0..32, so the range [33, 37) is fully masked for it.
    assert np.isneginf(ms[-1][0]).all()
    np.testing.assert_allclose(merge_partials(ms, ls, accs), attention(q, k, v), rtol=0, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(11)
    q, k, v = _random_case(rng, 3, 20, 8, 2, 6)
    k_rep = np.repeat(k, 4, axis=1)    # KV head g serves query heads 4g .. 4g+3
    v_rep = np.repeat(v, 4, axis=1)
    np.testing.assert_allclose(attention(q, k, v), attention(q, k_rep, v_rep), rtol=0, atol=1e-14)


def test_head_grouping_is_contiguous():
    # KV head g stores constant value g+1: query head h must read h // G + 1.
    kv_len, hkv, group, d = 5, 3, 4, 2
    keys = np.zeros((kv_len, hkv, d))
    values = np.broadcast_to(np.arange(1.0, hkv + 1)[None, :, None], (kv_len, hkv, d)).copy()
    out = attention(np.zeros((1, hkv * group, d)), keys, values)
    assert out[0, :, 0].tolist() == [h // group + 1.0 for h in range(hkv * group)]


def test_chunked_prefill_equals_one_shot():
    rng = np.random.default_rng(13)
    kv_len, q_len = 40, 24
    q, k, v = _random_case(rng, q_len, kv_len, 4, 2, 8)
    whole = attention(q, k, v)
    chunks = []
    for a in range(0, q_len, 7):
        b = min(q_len, a + 7)
        seen = kv_len - q_len + b           # cache length when this chunk runs
        chunks.append(attention(q[a:b], k[:seen], v[:seen]))
    np.testing.assert_allclose(np.concatenate(chunks), whole, rtol=0, atol=1e-13)


def test_decode_equals_last_prefill_row():
    rng = np.random.default_rng(17)
    q, k, v = _random_case(rng, 6, 15, 4, 4, 8)
    np.testing.assert_allclose(attention(q[-1:], k, v)[0], attention(q, k, v)[-1], rtol=0, atol=1e-14)


def test_single_visible_key_returns_its_value():
    rng = np.random.default_rng(19)
    q, k, v = _random_case(rng, 5, 5, 2, 1, 4, scale=10.0)
    out = attention(q, k, v)
    assert (out[0] == v[0][[0, 0]]).all()


def test_errors():
    z = np.zeros
    with pytest.raises(ValueError):
        attention(z((1, 2, 4)), z((0, 1, 4)), z((0, 1, 4)))       # empty cache
    with pytest.raises(ValueError):
        attention(z((3, 2, 4)), z((2, 1, 4)), z((2, 1, 4)))       # q_len > kv_len
    with pytest.raises(ValueError):
        attention(z((1, 3, 4)), z((2, 2, 4)), z((2, 2, 4)))       # Hq % Hkv != 0


# ------------------------------------------------------------ paged == logical
def _build(wl, order=None):
    pool = Pool(wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim,
                allocation_order=wl.allocation_order if order is None else order)
    for op in append_stream(wl):
        if op[0] == "create":
            pool.create(op[1])
        elif op[0] == "share":
            pool.share(op[1], op[2], op[3])
        else:
            _, s, n, k, v = op
            slots = pool.append(s, n)
            pool.write(slots, wl.to_f64(k), wl.to_f64(v))
        pool.validate()
    return pool


def test_paged_gather_equals_logical_rows_and_relabel_invariance():
    wl = prefix_prefill(batch=3, prefix=37, chunk=11, num_blocks=64, num_heads=4,
                        num_kv_heads=2, head_dim=8, block_size=4)
    pool = _build(wl)
    pool2 = _build(wl, order=list(range(wl.num_blocks))[::-1])
    rows = logical_kv(wl, [0, 1, 2])
    for s in range(3):
        k, v = pool.gather(s)
        np.testing.assert_array_equal(k, wl.to_f64(rows[s][0]))
        np.testing.assert_array_equal(v, wl.to_f64(rows[s][1]))
        k2, v2 = pool2.gather(s)
        np.testing.assert_array_equal(k, k2)
        np.testing.assert_array_equal(v, v2)
    assert pool.page_table(0)[:9] == pool.page_table(1)[:9]   # shared complete blocks
    assert pool.refs[pool.page_table(0)[0]] == 3


def test_shared_prefix_same_query_same_output():
    wl = prefix_prefill(batch=2, prefix=13, chunk=0, num_blocks=16, num_heads=4,
                        num_kv_heads=2, head_dim=8, block_size=4)
    pool = _build(wl)
    q = np.random.default_rng(3).standard_normal((2, 4, 8))
    assert (paged_attention(pool, 0, q) == paged_attention(pool, 1, q)).all()


def test_tiny_workload_paged_equals_brute_force():
    wl = tiny_fp32()
    pool = _build(wl)
    assert pool.page_table(0) == (2, 4) and pool.page_table(1) == (2, 3, 6)
    rows = logical_kv(wl, [0, 1])
    q = np.random.default_rng(0).standard_normal((3, 1, 8))
    for s in (0, 1):
        kv = [wl.to_f64(x) for x in rows[s]]
        np.testing.assert_allclose(paged_attention(pool, s, q[:1]), brute_force_attention(q[:1], *kv), atol=1e-14)
    np.testing.assert_allclose(paged_attention(pool, 1, q), brute_force_attention(q, *[wl.to_f64(x) for x in rows[1]]), atol=1e-14)


# ------------------------------------------------------------ planted mistakes
def _mutant_no_scale(q, k, v):
    return attention(q * math.sqrt(q.shape[2]), k, v)


def _mutant_top_left_mask(q, k, v):
    q_len, kv_len = q.shape[0], k.shape[0]
    out = np.empty_like(q)
    for t in range(q_len):
        out[t] = attention(q[t:t + 1], k[:t + 1], v[:t + 1])[0]
    return out


def _mutant_interleaved_groups(q, k, v):
    hq, hkv = q.shape[1], k.shape[1]
    idx = [h % hkv for h in range(hq)]
    return attention(q, np.repeat(k, 1, axis=1)[:, idx], v[:, idx]) if hq != hkv else attention(q, k, v)


def test_pins_reject_planted_mistakes():
    keys, values, q = _causal_case()
    ref = attention(q, keys, values)
    assert not np.allclose(_mutant_no_scale(q, keys, values), ref, atol=1e-6)
    rng = np.random.default_rng(23)
    q2, k2, v2 = _random_case(rng, 3, 8, 4, 2, 4)
    assert not np.allclose(_mutant_top_left_mask(q2, k2, v2), brute_force_attention(q2, k2, v2), atol=1e-6)
    kv_len, hkv, group, d = 5, 2, 2, 2
    vals = np.broadcast_to(np.arange(1.0, hkv + 1)[None, :, None], (kv_len, hkv, d)).copy()
    out = _mutant_interleaved_groups(np.zeros((1, 4, d)), np.zeros((kv_len, hkv, d)), vals)
    assert out[0, :, 0].tolist() != [h // group + 1.0 for h in range(4)]
