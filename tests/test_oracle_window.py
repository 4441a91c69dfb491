"""Pins of the oracle's sliding window with sinks (oracle.window) and of the
pool's page-granular eviction.

Source: vladkulikov.com notebook "Модуль 10", eviction cell and explicit
window caches (tests/golden/p2_eviction.json).

* The notebook's streaming keep set for 16 tokens, budget 8, 4 sinks, and
  its consistency with the printed heavy hitters and lost heavy hitters.
* The notebook's window-3 cache: after five single-token appends the
  retained interval is [2, 5); rollback to 4 is accepted, to -1, 1 or 6
  refused; rollback to 2 then one append leaves [2, 3).  (With block size 1
  page granularity is token granularity.)
* The notebook's check that attention over the window-3 cache equals
  attention over keys [max(0, step - 2), step], at block sizes 1 and 2.
* Brute force: with every row resident, windowed attention equals attention
  over the index set {p < n : p < sinks or p >= n - recent} (all of [0, n)
  when n <= sinks + recent), for random shapes, multi-row queries included.
* Closed-form page counts of a long windowed sequence, pool invariants,
  fork / share of a windowed sequence.
* Planted mistakes (a window one token too wide, sinks ignored, releasing
  the page of the first appended row) each fail a pin.
"""

import json
import os

import numpy as np
import pytest

from oracle import Pool, attention, brute_force_attention, window_keep, windowed_attention
from oracle.pool import HOLE

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "p2_eviction.json")


def test_notebook_streaming_keep_set():
    g = json.load(open(GOLDEN))
    n = len(g["attention_mass"])
    sinks = g["sink_tokens"]
    keep = window_keep(n, sinks, g["budget"] - sinks)
    assert list(keep) == g["streaming"]
    assert sorted(set(g["heavy_hitters"]) - set(keep)) == g["lost_heavy_hitters"]
    assert window_keep(5, 4, 4) == (0, 1, 2, 3, 4)
    assert window_keep(9, 0, 8) == tuple(range(1, 9))
    assert window_keep(9, 8, 0) == tuple(range(8))
    # The budget always holds exactly min(length, budget) positions.
    for length in range(12):
        for s in range(5):
            for r in range(5):
                if s + r:
                    assert len(window_keep(length, s, r)) == min(length, s + r)
    with pytest.raises(ValueError):  # sinks above the budget: a negative recent part
        window_keep(9, 5, -1)
    with pytest.raises(ValueError):
        window_keep(9, 0, 0)


def _window_pool(bs, recent, sinks=0, nb=64, d=2):
    pool = Pool(nb, bs, 1, d)
    pool.create(0)
    pool.set_window(0, sinks, recent)
    return pool


def test_notebook_window_cache_intervals():
    w = json.load(open(GOLDEN))["window_cache"]
    pool = _window_pool(1, w["window"])
    for value in range(w["appends"]):
        slots = pool.append(0, 1)
        pool.write(slots, np.full((1, 1, 2), value), np.full((1, 1, 2), value + 100))
    assert (pool.evicted_end(0), pool.sequence_length(0)) == (w["start_pos_after"], w["next_pos_after"])
    pos, keys, _ = pool.resident(0)
    assert pos == [2, 3, 4] and keys[:, 0, 0].tolist() == [2, 3, 4]
    for bad in w["invalid_rollbacks"]:
        with pytest.raises(ValueError):
            pool.truncate(0, bad)
    assert (pool.evicted_end(0), pool.sequence_length(0)) == (2, 5)
    pool.truncate(0, w["valid_rollback"])
    assert pool.resident(0)[0] == [2, 3]
    pool.truncate(0, 2)
    assert pool.resident(0)[0] == []
    pool.append(0, 1)
    assert [pool.evicted_end(0), pool.sequence_length(0)] == w["rollback_to_start_then_append_one"]
    assert pool.resident(0)[0] == [2]
    pool.validate()


@pytest.mark.parametrize("bs", [1, 2])
def test_notebook_window_attention_equals_slice(bs):
    rng = np.random.default_rng(17)
    keys = rng.standard_normal((6, 1, 4))
    values = rng.standard_normal((6, 1, 4))
    queries = rng.standard_normal((6, 1, 4))
    pool = Pool(16, bs, 1, 4)
    pool.create(0)
    pool.set_window(0, 0, 3)
    for step in range(6):
        pool.write(pool.append(0, 1), keys[step:step + 1], values[step:step + 1])
        pos, k, v = pool.resident(0)
        got = windowed_attention(queries[step:step + 1], k, v, pos, step + 1, 0, 3)
        lo = max(0, step - 2)
        want = attention(queries[step:step + 1], keys[lo:step + 1], values[lo:step + 1])
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    pool.validate()


@pytest.mark.parametrize("seed", range(4))
def test_windowed_attention_brute_force(seed):
    rng = np.random.default_rng(seed)
    for _ in range(6):
        n = int(rng.integers(1, 40))
        sinks = int(rng.integers(0, 6))
        recent = int(rng.integers(0 if sinks else 1, 12))
        q_len = int(rng.integers(1, min(n, 5) + 1))
        keys = rng.standard_normal((n, 2, 3))
        values = rng.standard_normal((n, 2, 3))
        q = rng.standard_normal((q_len, 4, 3))
        got = windowed_attention(q, keys, values, range(n), n, sinks, recent)
        for t in range(q_len):
            m = n - q_len + t + 1
            idx = list(range(m)) if m <= sinks + recent else [p for p in range(m) if p < sinks or p >= m - recent]
            want = brute_force_attention(q[t:t + 1], keys[idx], values[idx])
            np.testing.assert_allclose(got[t:t + 1], want, rtol=1e-10, atol=1e-12)


def test_page_granular_eviction_counts():
    bs, sinks, recent, n = 4, 5, 10, 100
    pool = _window_pool(bs, recent, sinks, nb=40)
    for p in range(n):
        pool.append(0, 1)
        pool.validate()
    table = pool.tables[0]
    # Last append: first new row 99 sees [90, 99]; pages [2, 22) lie wholly
    # between the sink pages (positions 0..7) and position 88.
    assert [j for j, b in enumerate(table) if b == HOLE] == list(range(2, 22))
    assert len(pool.free) == 40 - 5
    assert pool.evicted_end(0) == 88
    # A multi-token append keeps every page its first row still needs.
    pool.append(0, 8)                     # rows 100..107; row 100 sees [91, 100]
    assert [j for j, b in enumerate(table) if b == HOLE] == list(range(2, 22))
    pool.append(0, 1)                     # row 108 sees [99, 108]: pages 22, 23 go
    assert [j for j, b in enumerate(table) if b == HOLE] == list(range(2, 24))
    # Fork and share copy the holes and the window.
    pool.fork(0, 1)
    pool.share(0, 2, 96)
    assert pool.windows[1] == pool.windows[2] == (sinks, recent)
    assert pool.tables[2] == table[:24]
    pool.validate()
    pool.release(0)
    pool.release(1)
    pool.release(2)
    assert len(pool.free) == 40
    pool.validate()


def test_recent_zero_keeps_the_appended_pages():
    pool = _window_pool(2, 0, sinks=2, nb=16)
    for _ in range(9):
        pool.append(0, 1)
        pool.validate()
        assert pool.tables[0][-1] != HOLE
    assert window_keep(9, 2, 0) == (0, 1)


# ------------------------------------------------------------ planted mistakes
def _mutant_wide(length, budget, sinks):
    return window_keep(length, sinks, budget - sinks + 1) if length > budget else tuple(range(length))


def _mutant_no_sinks(length, budget, sinks):
    return window_keep(length, 0, budget)


def test_pins_reject_planted_mistakes():
    g = json.load(open(GOLDEN))
    n = len(g["attention_mass"])
    assert list(_mutant_wide(n, g["budget"], g["sink_tokens"])) != g["streaming"]
    assert list(_mutant_no_sinks(n, g["budget"], g["sink_tokens"])) != g["streaming"]
    # Releasing the page of the first appended row (end = lo // bs only):
    # with recent 0 the tail page itself would be released.
    first_new, recent, bs = 3, 0, 2
    lo = first_new + 1 - recent
    assert lo // bs > first_new // bs        # the mutant's end covers page 1 (rows 2, 3)
    assert min(lo // bs, first_new // bs) == first_new // bs
