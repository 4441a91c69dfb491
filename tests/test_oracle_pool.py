"""Pins of the oracle's pool model against what the pages fix.

* The printed allocation trace of the "Модуль 10" notebook's ``PagedKVPool``
  demo (embedded reference contract, entry ``paged.trace``), stored in
  ``tests/golden/p2_paged_trace.json``.
* The same trace under another allocation order: tables are the identity-
  order tables relabelled through the permutation.
* The ownership trace of abhik.ai "examples/pagedattention.py"
  (``ownership_trace``: 7-token prompt, fork, COW append, private append,
  boundary append, two releases) -- the page prints no values; the expected
  tables below were worked out by hand from its rules.
* The notebook's negative tests (unknown / duplicate ids, preflighted OOM
  leaves the state unchanged, prefix longer than the source, unequal-prefix
  release and COW payloads, zero waste at 2048 tokens / block 16) and its
  lecture-core private-page test.
* The first-free-in-order rule against a literal scan of the order.
"""

import json
import os

import numpy as np
import pytest

from oracle import Pool, OutOfBlocks, UnknownSequence, SequenceExists

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "p2_paged_trace.json")
A, B = 0, 1
NAMES = {A: "A", B: "B"}


def _p2_demo(order=None):
    pool = Pool(8, 4, allocation_order=order, store_values=False)
    snaps = {}
    pool.create(A)
    pool.append(A, 6)
    snaps["after_a"] = pool.snapshot(NAMES)
    pool.share(A, B, 6)
    snaps["after_share"] = pool.snapshot(NAMES)
    pool.append(B, 3)
    snaps["after_b_append"] = pool.snapshot(NAMES)
    cow_ok = pool.page_table(A)[-1] != pool.page_table(B)[1]
    pool.release(A)
    snaps["after_a_release"] = pool.snapshot(NAMES)
    pool.validate()
    return pool, snaps, cow_ok


def test_printed_trace_matches_golden():
    golden = json.load(open(GOLDEN))["trace"]
    _, snaps, cow_ok = _p2_demo()
    assert cow_ok
    for event, expected in golden.items():
        assert snaps[event] == expected, event


def test_printed_trace_relabelled_by_permutation():
    golden = json.load(open(GOLDEN))["trace"]
    order = [2, 4, 3, 6, 5, 0, 1, 7]   # default_rng(0).permutation(8)
    pool, snaps, cow_ok = _p2_demo(order)
    assert cow_ok
    for event, expected in golden.items():
        got = snaps[event]
        for key, value in expected.items():
            if key == "sequences":
                for name, entry in value.items():
                    assert got["sequences"][name]["length"] == entry["length"]
                    assert got["sequences"][name]["blocks"] == [order[b] for b in entry["blocks"]]
            else:
                assert got[key] == value, (event, key)


def test_tiny_workload_tables_slots_refcounts():
    order = [2, 4, 3, 6, 5, 0, 1, 7]
    pool = Pool(8, 4, allocation_order=order, store_values=False)
    pool.create(A)
    slots_a = pool.append(A, 6)
    pool.share(A, B, 6)
    slots_b = pool.append(B, 3)
    assert pool.page_table(A) == (2, 4)
    assert pool.page_table(B) == (2, 3, 6)
    assert slots_a == [8, 9, 10, 11, 16, 17]
    # B's own tokens 6, 7 land in the COW copy (block 3), token 8 in block 6.
    assert slots_b == [14, 15, 24]
    assert [pool.slot(B, p) for p in range(9)] == [8, 9, 10, 11, 12, 13, 14, 15, 24]
    assert pool.copies == [(4, 3)]
    refs = [0] * 8
    refs[2], refs[4], refs[3], refs[6] = 2, 1, 1, 1
    assert pool.refs.tolist() == refs
    pool.validate()


def test_first_page_ownership_trace_by_hand():
    order = [5, 2, 7, 0, 3, 6, 1, 4]
    pool = Pool(8, 4, num_kv_heads=1, head_dim=3, allocation_order=order)

    def waste():
        return pool.stats()["internal_waste_tokens"]

    pool.create(A)
    for _ in range(7):
        pool.append(A, 1)
    assert pool.page_table(A) == (5, 2) and waste() == 1
    pool.fork(A, B)
    assert pool.page_table(B) == (5, 2) and pool.refs[5] == 2 and pool.refs[2] == 2
    assert waste() == 1
    pool.append(B, 1)                    # B's 8th token: copy-on-write of block 2
    assert pool.page_table(B) == (5, 7) and pool.copies == [(2, 7)] and waste() == 1
    pool.append(A, 1)                    # A's 8th token: block 2 is private again
    assert pool.page_table(A) == (5, 2) and waste() == 0
    pool.append(B, 1)                    # B's 9th token: block boundary
    assert pool.page_table(B) == (5, 7, 0) and waste() == 3
    pool.release(A)
    assert sorted(pool.free) == [1, 2, 3, 4, 6]
    pool.release(B)
    assert sorted(pool.free) == list(range(8))   # the full pool is recovered
    pool.validate()


def test_negative_contract():
    pool = Pool(2, 4, store_values=False)
    with pytest.raises(KeyError):
        pool.append("missing", 1)
    pool.create("x")
    with pytest.raises(ValueError):
        pool.create("x")
    pool.append("x", 6)
    before = pool.snapshot()
    refs_before = pool.refs.copy()
    with pytest.raises(MemoryError):
        pool.append("x", 3)
    assert pool.snapshot() == before and (pool.refs == refs_before).all()
    with pytest.raises(ValueError):
        pool.share("x", "y", 7)
    assert "y" not in pool.tables
    pool.validate()
    assert issubclass(OutOfBlocks, MemoryError)
    assert issubclass(UnknownSequence, KeyError)
    assert issubclass(SequenceExists, ValueError)


@pytest.mark.parametrize("action", ["release", "append"])
def test_short_child_survives_parent(action):
    pool = Pool(4, 4, store_values=False)
    pool.create("parent")
    pool.append("parent", 3)
    pool.share("parent", "child", 1)
    if action == "release":
        pool.release("parent")
        assert pool.stats()["physical_payload_tokens"] == 1
    else:
        pool.append("parent", 1)
        assert pool.stats()["physical_payload_tokens"] == 5
    pool.append("child", 2)
    pool.validate()


def test_exact_fill_has_no_waste():
    pool = Pool(128, 16, store_values=False)
    pool.create("fixed")
    pool.append("fixed", 2048)
    assert pool.stats()["internal_waste_tokens"] == 0
    golden = json.load(open(GOLDEN))["other_values"]
    assert golden["exact_2048_waste_fraction"] == 0.0


def test_private_pages_lecture_core():
    pool = Pool(128, 16, store_values=False)
    pool.create("a")
    pool.append("a", 2048)
    assert len(pool.page_table("a")) == 128
    before = (sorted(pool.free), dict(pool.lengths), {k: list(v) for k, v in pool.tables.items()})
    with pytest.raises(MemoryError):
        pool.append("a", 1)
    assert before == (sorted(pool.free), dict(pool.lengths), {k: list(v) for k, v in pool.tables.items()})
    pool.release("a")
    assert len(pool.free) == 128


def test_zero_token_append_on_shared_tail_copies_nothing():
    pool = Pool(4, 4, store_values=False)
    pool.create(A)
    pool.append(A, 2)
    pool.fork(A, B)
    assert pool.append(B, 0) == []
    assert pool.copies == [] and pool.page_table(B) == pool.page_table(A)


def test_full_shared_tail_needs_no_copy():
    pool = Pool(4, 4, store_values=False)
    pool.create(A)
    pool.append(A, 4)
    pool.fork(A, B)
    pool.append(B, 1)
    assert pool.copies == [] and pool.page_table(B)[0] == pool.page_table(A)[0]
    assert pool.refs[pool.page_table(A)[0]] == 2


def test_allocation_is_first_free_in_order_literal_scan():
    rng = np.random.default_rng(123)
    for trial in range(20):
        n = int(rng.integers(4, 24))
        bs = int(rng.integers(1, 6))
        order = [int(x) for x in rng.permutation(n)]
        pool = Pool(n, bs, allocation_order=order, store_values=False)
        live = []
        next_id = 0
        for step in range(60):
            kind = rng.integers(0, 4)
            free_before = set(pool.free)
            tables_before = {s: list(t) for s, t in pool.tables.items()}
            try:
                if kind == 0 or not live:
                    pool.create(next_id)
                    live.append(next_id)
                    next_id += 1
                elif kind == 1:
                    s = live[int(rng.integers(len(live)))]
                    pool.append(s, int(rng.integers(0, 3 * bs)))
                elif kind == 2:
                    s = live[int(rng.integers(len(live)))]
                    pool.share(s, next_id, int(rng.integers(0, pool.lengths[s] + 1)))
                    live.append(next_id)
                    next_id += 1
                else:
                    s = live.pop(int(rng.integers(len(live))))
                    pool.release(s)
            except MemoryError:
                assert set(pool.free) == free_before
                assert {s: list(t) for s, t in pool.tables.items()} == tables_before
            newly = [b for b in range(n) if b in free_before and b not in pool.free]
            # Blocks taken by this step are exactly the first k free ids of the order.
            literal = [b for b in order if b in free_before][:len(newly)]
            assert sorted(newly) == sorted(literal)
            pool.validate()
