"""Sliding windows with sinks and rollback through the C ABI (host-only
calls on metadata-only pools) against the oracle pool.

Source: vladkulikov.com notebook "Модуль 10", eviction cell and explicit
window caches.  Bar: bit-exact tables (released pages read -1), lengths,
refcounts, accounting, slots and allocation order.
"""

import copy
import json
import os

import numpy as np
import pytest

import oracle
from oracle.pool import HOLE
from paged_kv_cache_block_amd import DevicePool
from paged_kv_cache_block_amd.abi import (InvalidArgumentError, OutOfBlocksError,
                                          UnknownSequenceError)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "p2_eviction.json")


def _same(pool, ref):
    ids = sorted(ref.tables)
    assert pool.sequences().tolist() == ids
    for s in ids:
        assert pool.block_table(s).tolist() == ref.tables[s], s
        assert pool.seq_len(s) == ref.lengths[s]
    assert [pool.refcount(b) for b in range(ref.num_blocks)] == ref.refs.tolist()
    assert pool.stats() == ref.stats()
    assert pool.pending_copies() == ref.copies
    pool.validate()
    ref.validate()


def test_notebook_window_cache_through_abi():
    w = json.load(open(GOLDEN))["window_cache"]
    pool = DevicePool(16, 1, 1, 16, metadata_only=True)
    pool.create(0)
    pool.set_window(0, 0, w["window"])
    for _ in range(w["appends"]):
        pool.append(0, 1)
    table = pool.block_table(0).tolist()
    start = max(j for j, b in enumerate(table) if b == HOLE) + 1
    assert (start, pool.seq_len(0)) == (w["start_pos_after"], w["next_pos_after"])
    for bad in w["invalid_rollbacks"]:
        with pytest.raises(InvalidArgumentError):
            pool.truncate(0, bad)
    pool.truncate(0, w["valid_rollback"])
    pool.truncate(0, 2)
    pool.append(0, 1)
    assert pool.seq_len(0) == 3 and pool.block_table(0).tolist()[:2] == [HOLE, HOLE]
    pool.validate()


def test_window_argument_errors():
    pool = DevicePool(8, 4, 1, 16, metadata_only=True)
    pool.create(0)
    with pytest.raises(UnknownSequenceError):
        pool.set_window(5, 0, 4)
    for sinks, recent in ((0, 0), (-1, 4), (2, -1)):
        with pytest.raises(InvalidArgumentError):
            pool.set_window(0, sinks, recent)
    with pytest.raises(UnknownSequenceError):
        pool.truncate(5, 0)
    pool.append(0, 3)
    with pytest.raises(InvalidArgumentError):
        pool.truncate(0, 4)


@pytest.mark.parametrize("seed", range(8))
def test_differential_fuzz_against_oracle(seed):
    rng = np.random.default_rng(seed)
    bs = int(rng.choice([1, 2, 4, 16]))
    nb = 96
    order = rng.permutation(nb)
    pool = DevicePool(nb, bs, 1, 16, allocation_order=order, metadata_only=True)
    ref = oracle.Pool(nb, bs, allocation_order=order, store_values=False)
    live, next_id = [], 0
    for _ in range(250):
        op = rng.random()
        if op < 0.12 or not live:
            pool.create(next_id)
            ref.create(next_id)
            if rng.random() < 0.7:
                sinks = int(rng.integers(0, 6))
                recent = int(rng.integers(0 if sinks else 1, 24))
                pool.set_window(next_id, sinks, recent)
                ref.set_window(next_id, sinks, recent)
            live.append(next_id)
            next_id += 1
        elif op < 0.55:
            s = live[int(rng.integers(0, len(live)))]
            n = int(rng.integers(0, 12))
            try:
                want = ref.append(s, n)
            except oracle.OutOfBlocks:
                with pytest.raises(OutOfBlocksError):
                    pool.append(s, n)
            else:
                assert pool.append(s, n).tolist() == want
        elif op < 0.7:
            batch = [live[int(i)] for i in rng.integers(0, len(live), size=int(rng.integers(1, 4)))]
            ns = [int(x) for x in rng.integers(0, 20, size=len(batch))]
            snap = (pool.stats(), {s: pool.block_table(s).tolist() for s in live})
            # All or nothing: the oracle replays the batch on a copy first.
            trial = copy.deepcopy(ref)
            ok, want = True, []
            for s, n in zip(batch, ns):
                try:
                    want += trial.append(s, n)
                except oracle.OutOfBlocks:
                    ok = False
                    break
            if ok:
                assert pool.append_batch(batch, ns).tolist() == want
                ref = trial
            else:
                with pytest.raises(OutOfBlocksError):
                    pool.append_batch(batch, ns)
                assert snap == (pool.stats(), {s: pool.block_table(s).tolist() for s in live})
        elif op < 0.78:
            s = live[int(rng.integers(0, len(live)))]
            n = ref.lengths[s]
            new_len = int(rng.integers(0, n + 1))
            try:
                ref.truncate(s, new_len)
            except ValueError:
                with pytest.raises(InvalidArgumentError):
                    pool.truncate(s, new_len)
            else:
                pool.truncate(s, new_len)
        elif op < 0.86:
            s = live[int(rng.integers(0, len(live)))]
            prefix = int(rng.integers(0, ref.lengths[s] + 1))
            try:
                ref.share(s, next_id, prefix)
            except ValueError:
                with pytest.raises(InvalidArgumentError):
                    pool.share(s, next_id, prefix)
            else:
                pool.share(s, next_id, prefix)
                live.append(next_id)
                next_id += 1
        else:
            s = live.pop(int(rng.integers(0, len(live))))
            pool.release(s)
            ref.release(s)
        _same(pool, ref)
        # The next block each would hand out is the same.
        assert pool.stats()["free_blocks"] == len(ref.free)
