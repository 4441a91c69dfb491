"""Pins of the oracle's prefix-hash block reuse (oracle.prefix) and of the
pool's pins / adopt.

Source: vladkulikov.com notebook "Модуль 10", prefix-caching cell.

* The notebook's asserted trace results (tests/golden/p2_prefix_trace.json):
  with one shared scope 98% of the 500 requests hit and 490 * 32 of the
  500 * 48 input tokens are reused; with one scope per user 80% hit.
* Closed forms of the same trace: the isolated scope reuses 400 * 32 tokens;
  the cache ends with 10 + 10 + 500 keys (shared) and 100 * 7 (isolated),
  one pinned block each.
* The notebook's identity checks: equal block content after different
  preceding tokens, or under another revision, gives different keys.
* Brute force on small random traces: the hit equals the longest common
  block-aligned prefix with any earlier request of the same scope and
  revision (what a set of all-preceding-token keys means).
* Pool invariants hold throughout (refcount = table references + pins), and
  ``clear`` returns every pinned block.
* Planted mistakes (a key of the block's own tokens only, a hit that does not
  stop at the first miss) each fail a pin.
"""

import json
import os

import numpy as np
import pytest

from oracle import Pool, PrefixCache, block_key, run_prefix_trace
from synth import prefix_trace_requests

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "p2_prefix_trace.json")


def _trace(isolated, num_blocks=1024):
    reqs = prefix_trace_requests()
    pool = Pool(num_blocks, 16, store_values=False)
    scope_of = (lambda i: reqs[i][0]) if isolated else (lambda i: "shared-public-template")
    hit_frac, reuse, cache = run_prefix_trace(pool, [r[2] for r in reqs], scope_of)
    return hit_frac, reuse, cache, pool


def test_notebook_trace_fractions():
    gold = json.load(open(GOLDEN))
    hit, reuse, cache, pool = _trace(False)
    assert np.isclose(hit, gold["shared_scope"]["hit_request_fraction"])
    assert np.isclose(reuse, eval(gold["shared_scope"]["reused_input_fraction_expr"], {}))
    assert len(cache.entries) == 10 + 10 + 500
    pool.validate()
    assert pool.pins.sum() == 520 and not pool.tables
    hit, reuse, cache, pool = _trace(True)
    assert np.isclose(hit, gold["isolated_scope"]["hit_request_fraction"])
    assert np.isclose(reuse, 400 * 32 / (500 * 48))
    assert len(cache.entries) == 100 * 7
    pool.validate()
    assert cache.clear() == 700
    assert len(pool.free) == pool.num_blocks and pool.pins.sum() == 0
    pool.validate()


def test_notebook_key_identity():
    a = list(range(32))
    b = a.copy()
    b[0] = 999
    assert a[16:32] == b[16:32]
    assert block_key("scope", "r1", a, 32) != block_key("scope", "r1", b, 32)
    assert block_key("scope", "r1", a, 32) != block_key("scope", "r2", a, 32)
    # ... and through a cache: the second block of b is not found after a.
    pool = Pool(16, 16, store_values=False)
    cache = PrefixCache(pool)
    pool.create("a")
    pool.append("a", 32)
    cache.register("a", a, "scope", "r1")
    assert cache.lookup(a, "scope", "r1") == 32
    assert cache.lookup(b, "scope", "r1") == 0
    assert cache.lookup(a, "scope", "r2") == 0
    assert cache.lookup(a[:16] + b[16:], "scope", "r1") == 32
    assert cache.lookup(a[:16] + [5] * 16, "scope", "r1") == 16
    assert cache.lookup(a[:31], "scope", "r1") == 16     # only complete blocks


def test_attach_shares_blocks_and_appends_after_them():
    pool = Pool(32, 4, store_values=False)
    cache = PrefixCache(pool)
    toks = list(range(10))
    pool.create(0)
    pool.append(0, 10)
    assert cache.register(0, toks, "s", "r") == 2          # blocks ending at 4 and 8
    assert cache.register(0, toks, "s", "r") == 0
    hit = cache.attach(1, toks[:9] + [77], "s", "r")
    assert hit == 8 and pool.tables[1] == pool.tables[0][:2]
    assert [pool.refs[b] for b in pool.tables[0]] == [3, 3, 1]   # seq 0, seq 1, the pin
    slots = pool.append(1, 2)                               # new block, no copy-on-write
    assert pool.copies == [] and slots[0] // 4 not in pool.tables[0]
    pool.release(0)
    pool.release(1)
    pool.validate()
    assert [pool.refs[b] for b in range(32) if pool.refs[b]] == [1, 1]
    hit = cache.attach(2, toks, "s", "r")
    assert hit == 8 and pool.sequence_length(2) == 8
    pool.validate()


def _brute_hit(history, tokens, bs):
    best = 0
    for prev in history:
        n = 0
        while n + bs <= min(len(prev), len(tokens)) and prev[:n + bs] == tokens[:n + bs]:
            n += bs
        best = max(best, n)
    return best


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_hits_equal_brute_force_on_random_traces(seed):
    rng = np.random.default_rng(seed)
    bs = 4
    pool = Pool(4096, bs, store_values=False)
    cache = PrefixCache(pool)
    history = {}
    for i in range(60):
        scope = int(rng.integers(0, 3))
        rev = "r" + str(int(rng.integers(0, 2)))
        base = [int(x) for x in rng.integers(0, 3, size=int(rng.integers(1, 30)))]
        tokens = base
        hist = history.setdefault((scope, rev), [])
        assert cache.lookup(tokens, scope, rev) == _brute_hit(hist, tokens, bs)
        hit = cache.attach(i, tokens, scope, rev)
        pool.append(i, len(tokens) - hit)
        cache.register(i, tokens, scope, rev)
        if rng.random() < 0.5:
            pool.release(i)
        hist.append(tokens)
        pool.validate()


# ------------------------------------------------------------ planted mistakes
def _mutant_block_only_key(tokens, end, scope, revision, bs=16):
    return (scope, revision, tuple(tokens[end - bs:end]))


def _mutant_no_stop_lookup(cache, tokens, scope, rev):
    bs = cache.pool.block_size
    hit = 0
    for end in range(bs, len(tokens) + 1, bs):
        if block_key(scope, rev, tokens, end) in cache.entries:
            hit = end
    return hit


def test_pins_reject_planted_mistakes():
    # A key of the block's own tokens: the notebook's context-identity check fails.
    a = list(range(32))
    b = a.copy()
    b[0] = 999
    assert _mutant_block_only_key(a, 32, "scope", "r1") == _mutant_block_only_key(b, 32, "scope", "r1")
    assert block_key("scope", "r1", a, 32) != block_key("scope", "r1", b, 32)
    # A walk that does not stop at the first miss: the brute-force pin fails.
    pool = Pool(16, 16, store_values=False)
    cache = PrefixCache(pool)
    pool.create(0)
    pool.append(0, 48)
    toks = list(range(48))
    cache.register(0, toks, "s", "r")
    del cache.entries[block_key("s", "r", toks, 16)]
    assert _mutant_no_stop_lookup(cache, toks, "s", "r") == 48
    assert cache.lookup(toks, "s", "r") == 0 == _brute_hit([], toks, 16)
