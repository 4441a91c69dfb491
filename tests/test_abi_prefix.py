"""Prefix-hash block reuse through the C ABI (host-only calls, metadata-only
pools) against the oracle's PrefixCache.

Source: vladkulikov.com notebook "Модуль 10", prefix-caching cell.  Bar:
bit-exact hits, block tables, refcounts, accounting and key counts.
"""

import json
import os

import numpy as np
import pytest

import oracle
from oracle import PrefixCache
from paged_kv_cache_block_amd import DevicePool
from paged_kv_cache_block_amd.abi import (InvalidArgumentError, SequenceExistsError,
                                          UnknownSequenceError)
from synth import prefix_trace_requests

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "p2_prefix_trace.json")


def _same_state(pool, ref, seqs):
    for s in seqs:
        assert pool.block_table(s).tolist() == ref.tables[s]
        assert pool.seq_len(s) == ref.lengths[s]
    assert [pool.refcount(b) for b in range(ref.num_blocks)] == ref.refs.tolist()
    assert pool.stats() == ref.stats()
    pool.validate()
    ref.validate()


@pytest.mark.parametrize("isolated", [False, True], ids=["shared", "isolated"])
def test_notebook_trace_through_abi(isolated):
    gold = json.load(open(GOLDEN))
    reqs = prefix_trace_requests()
    order = np.random.default_rng(4).permutation(1024)
    pool = DevicePool(1024, 16, 1, 16, allocation_order=order, metadata_only=True)
    ref = oracle.Pool(1024, 16, allocation_order=order, store_values=False)
    cache = PrefixCache(ref)
    hits = cached = 0
    for i, (user, turn, tokens) in enumerate(reqs):
        scope = f"user-{user}" if isolated else "shared-public-template"
        assert pool.prefix_lookup(tokens, scope, "model-r1") == cache.lookup(tokens, scope, "model-r1")
        hit = pool.prefix_attach(i, tokens, scope, "model-r1")
        assert hit == cache.attach(i, tokens, scope, "model-r1")
        pool.append(i, len(tokens) - hit)
        ref.append(i, len(tokens) - hit)
        assert pool.prefix_register(i, tokens, scope, "model-r1") == cache.register(i, tokens, scope, "model-r1")
        if i % 97 == 0:
            _same_state(pool, ref, [i])
        pool.release(i)
        ref.release(i)
        hits += hit > 0
        cached += hit
    key = "isolated_scope" if isolated else "shared_scope"
    assert np.isclose(hits / 500, gold[key]["hit_request_fraction"])
    if not isolated:
        assert np.isclose(cached / (500 * 48), eval(gold[key]["reused_input_fraction_expr"], {}))
    assert pool.prefix_entries() == len(cache.entries) == (700 if isolated else 520)
    _same_state(pool, ref, [])
    assert pool.prefix_clear() == cache.clear()
    _same_state(pool, ref, [])
    assert pool.stats()["free_blocks"] == 1024


def test_key_identity_through_abi():
    pool = DevicePool(16, 16, 1, 16, metadata_only=True)
    a = list(range(32))
    b = a.copy()
    b[0] = 999
    pool.create(1)
    pool.append(1, 32)
    assert pool.prefix_register(1, a, "scope", "r1") == 2
    assert pool.prefix_lookup(a, "scope", "r1") == 32
    assert pool.prefix_lookup(b, "scope", "r1") == 0
    assert pool.prefix_lookup(a, "scope", "r2") == 0
    assert pool.prefix_lookup(a, "scope2", "r1") == 0
    assert pool.prefix_lookup(a[:31], "scope", "r1") == 16
    # A scope / revision pair cannot be spelled as another by moving bytes.
    assert pool.prefix_lookup(a, "scop", "er1") == 0


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_differential_fuzz_against_oracle(seed):
    rng = np.random.default_rng(seed)
    bs, nb = 4, 512
    order = rng.permutation(nb)
    pool = DevicePool(nb, bs, 1, 16, allocation_order=order, metadata_only=True)
    ref = oracle.Pool(nb, bs, allocation_order=order, store_values=False)
    cache = PrefixCache(ref)
    live = []
    for i in range(120):
        op = rng.random()
        if op < 0.55:
            scope, rev = f"s{int(rng.integers(0, 3))}", f"r{int(rng.integers(0, 2))}"
            tokens = [int(x) for x in rng.integers(0, 3, size=int(rng.integers(0, 26)))]
            hit = pool.prefix_attach(i, tokens, scope, rev)
            assert hit == cache.attach(i, tokens, scope, rev)
            extra = len(tokens) - hit
            pool.append(i, extra)
            ref.append(i, extra)
            n_reg = int(rng.integers(0, len(tokens) + 1))
            assert pool.prefix_register(i, tokens[:n_reg], scope, rev) == cache.register(i, tokens[:n_reg], scope, rev)
            live.append(i)
        elif op < 0.8 and live:
            s = live.pop(int(rng.integers(0, len(live))))
            pool.release(s)
            ref.release(s)
        elif op < 0.9 and live:
            s = live[int(rng.integers(0, len(live)))]
            pool.append(s, 3)
            ref.append(s, 3)
        elif op < 0.93:
            assert pool.prefix_clear() == cache.clear()
        _same_state(pool, ref, live)
        assert pool.prefix_entries() == len(cache.entries)


def test_prefix_errors_change_nothing():
    pool = DevicePool(8, 4, 1, 16, metadata_only=True)
    pool.create(0)
    pool.append(0, 9)
    pool.prefix_register(0, list(range(9)), "s", "r")
    before = (pool.stats(), pool.prefix_entries(), [pool.refcount(b) for b in range(8)])
    with pytest.raises(SequenceExistsError):
        pool.prefix_attach(0, list(range(9)), "s", "r")
    with pytest.raises(UnknownSequenceError):
        pool.prefix_register(5, list(range(4)), "s", "r")
    with pytest.raises(InvalidArgumentError):
        pool.prefix_register(0, list(range(10)), "s", "r")   # more tokens than the sequence has
    assert before == (pool.stats(), pool.prefix_entries(), [pool.refcount(b) for b in range(8)])
    # An empty request attaches an empty sequence.
    assert pool.prefix_attach(7, [], "s", "r") == 0 and pool.seq_len(7) == 0
