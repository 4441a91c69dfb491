"""The C ABI without a GPU: the library loads, exports every declared
symbol, and its host bookkeeping equals the oracle's bit for bit.

Bookkeeping calls (create / append / share / fork / release / inspection)
never touch the device, so a metadata-only pool exercises them here.
"""

import json
import os
import re

import numpy as np

import oracle
import pytest

from oracle import Pool
from paged_kv_cache_block_amd import abi, DevicePool
from paged_kv_cache_block_amd.abi import (InvalidArgumentError, OutOfBlocksError,
                                          SequenceExistsError, UnknownSequenceError)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedattn.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "p2_paged_trace.json")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = abi.load()
    names = declared_functions()
    assert len(names) >= 20
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(abi.SIGNATURES), "binding and header disagree"


def _meta(num_blocks, block_size, order=None, dtype="bf16"):
    return DevicePool(num_blocks, block_size, 2, 8, dtype=dtype, allocation_order=order,
                      metadata_only=True)


def test_printed_trace_through_the_abi():
    golden = json.load(open(GOLDEN))["trace"]
    pool = _meta(8, 4)
    names = {0: "A", 1: "B"}

    def snap():
        out = dict(pool.stats())
        out["sequences"] = {names[int(s)]: {"blocks": pool.block_table(int(s)).tolist(),
                                            "length": pool.seq_len(int(s))}
                            for s in pool.sequences()}
        return out

    pool.create(0)
    pool.append(0, 6)
    assert snap() == golden["after_a"]
    pool.share(0, 1, 6)
    assert snap() == golden["after_share"]
    pool.append(1, 3)
    assert snap() == golden["after_b_append"]
    assert pool.block_table(0)[-1] != pool.block_table(1)[1]
    assert pool.pending_copies() == [(1, 2)]
    pool.release(0)
    assert snap() == golden["after_a_release"]
    pool.validate()


def test_errors_leave_state_unchanged():
    pool = _meta(2, 4)
    with pytest.raises(UnknownSequenceError):
        pool.append(5, 1)
    with pytest.raises(KeyError):
        pool.release(5)
    pool.create(1)
    with pytest.raises(SequenceExistsError):
        pool.create(1)
    pool.append(1, 6)
    before = (pool.stats(), pool.block_table(1).tolist(), pool.seq_len(1))
    with pytest.raises(OutOfBlocksError):
        pool.append(1, 3)
    with pytest.raises(MemoryError):
        pool.append(1, 3)
    assert before == (pool.stats(), pool.block_table(1).tolist(), pool.seq_len(1))
    with pytest.raises(InvalidArgumentError):
        pool.share(1, 2, 7)
    with pytest.raises(InvalidArgumentError):
        pool.append(1, -1)
    with pytest.raises(ValueError):
        abi.pa_refcount(pool.handle, 2)
    assert 2 not in pool.sequences()
    pool.validate()
    pool.release(1)
    with pytest.raises(UnknownSequenceError):
        pool.release(1)


def test_bad_descriptors_and_orders():
    with pytest.raises(InvalidArgumentError):
        DevicePool(4, 4, 1, 8, allocation_order=[0, 1, 1, 2], metadata_only=True)
    with pytest.raises(InvalidArgumentError):
        DevicePool(4, 4, 1, 8, allocation_order=[0, 1, 2, 4], metadata_only=True)
    with pytest.raises(InvalidArgumentError):
        DevicePool(0, 4, 1, 8, metadata_only=True)
    with pytest.raises(InvalidArgumentError):
        DevicePool(4, 4, 1, 1024, metadata_only=True)
    assert abi.pa_pool_bytes(abi.make_desc(10, 16, 8, 128, abi.PA_DTYPE_BF16)) == 10 * 16 * 8 * 128 * 2
    assert abi.pa_pool_bytes(abi.make_desc(10, 16, 8, 0, abi.PA_DTYPE_BF16)) == 0


def test_int8_pool_descriptor():
    # Codes plus one fp32 scale per row: the packed size of the notebook's
    # KV-compression experiment (2 n d + 2 n 4 bytes for n rows of K and V).
    per_pool = abi.pa_pool_bytes(abi.make_desc(10, 16, 8, 128, abi.PA_DTYPE_I8))
    assert per_pool == 10 * 8 * (16 * 128 + 16 * 4)
    n_rows = 10 * 16 * 8
    assert 2 * per_pool == oracle.packed_bytes(n_rows, 128, 8)
    # The 8-bit float codes share the layout byte for byte.
    assert abi.pa_pool_bytes(abi.make_desc(10, 16, 8, 128, abi.PA_DTYPE_FP8)) == per_pool
    for bs, d in ((8, 128), (16, 40), (4, 8)):
        for dt, name in ((abi.PA_DTYPE_I8, "i8"), (abi.PA_DTYPE_FP8, "fp8")):
            assert abi.pa_pool_bytes(abi.make_desc(10, bs, 8, d, dt)) == 0
            with pytest.raises(InvalidArgumentError):
                DevicePool(10, bs, 1, d, dtype=name, metadata_only=True)
    assert abi.pa_pool_bytes(abi.make_desc(10, 16, 8, 128, 4)) == 0
    pool = DevicePool(8, 16, 2, 64, dtype="i8", metadata_only=True)
    pool.create(1)
    assert pool.append(1, 20).tolist() == list(range(32))[:20]


def test_device_calls_on_metadata_only_pool_are_rejected():
    pool = _meta(8, 4)
    pool.create(0)
    pool.append(0, 5)
    with pytest.raises(InvalidArgumentError):
        abi.pa_reshape_and_cache(pool.handle, 16, 16, 16, 1, None)
    with pytest.raises(InvalidArgumentError):
        abi.pa_decode(pool.handle, [0], 2, 256, 256, 256, 4096, None)
    with pytest.raises(InvalidArgumentError):
        abi.pa_prefill_chunk(pool.handle, [0], [2], 2, 256, 256, 256, 4096, None)
    # Flushing a metadata-only pool just drops the pending list.
    abi.pa_flush_copies(pool.handle, None)


def test_decode_step_argument_errors_change_nothing():
    pool = _meta(16, 4)
    pool.create(0)
    pool.append(0, 5)
    before = (pool.stats(), pool.block_table(0).tolist())
    with pytest.raises(InvalidArgumentError):
        abi.pa_decode_step(pool.handle, [0], 2, 256, 256, 256, 256, 256, 1 << 20, None)
    assert before == (pool.stats(), pool.block_table(0).tolist())
    h = pool.handle
    step = abi.pa_decode_step_workspace_bytes(h, [0, 0], 4)
    assert step >= abi.pa_decode_workspace_bytes(h, [0, 0], 4) > 0
    assert abi.pa_decode_step_workspace_bytes(h, [5], 4) == 0


def test_workspace_queries():
    pool = _meta(64, 4)
    for s, n in enumerate([3, 17, 40]):
        pool.create(s)
        pool.append(s, n)
    pool.create(9)
    h = pool.handle
    assert abi.pa_decode_workspace_bytes(h, [0, 1, 2], 4) % 256 == 0
    assert abi.pa_decode_workspace_bytes(h, [0, 1, 2], 4) > 0
    assert abi.pa_decode_workspace_bytes(h, [0, 77], 4) == 0     # unknown sequence
    assert abi.pa_decode_workspace_bytes(h, [0, 9], 4) == 0      # empty sequence
    assert abi.pa_decode_workspace_bytes(h, [0], 3) == 0         # 3 heads over 2 KV heads
    assert abi.pa_prefill_workspace_bytes(h, [1, 2], [17, 1], 2) > 0
    assert abi.pa_prefill_workspace_bytes(h, [1], [18], 2) == 0  # q_len > length
    assert abi.pa_prefill_workspace_bytes(h, [1], [0], 2) == 0
    # Multi-token step: sized for the lengths after appending q_lens tokens.
    assert abi.pa_verify_step_workspace_bytes(h, [0, 1], [4, 2], 4) > 0
    assert abi.pa_verify_step_workspace_bytes(h, [9], [3], 4) > 0     # empty before, 3 after
    assert abi.pa_verify_step_workspace_bytes(h, [0], [0], 4) == 0
    assert abi.pa_verify_step_workspace_bytes(h, [77], [1], 4) == 0


def test_verify_step_on_metadata_only_pool_changes_nothing():
    pool = _meta(16, 4)
    pool.create(0)
    pool.append(0, 5)
    before = (pool.stats(), pool.block_table(0).tolist())
    with pytest.raises(InvalidArgumentError):
        abi.pa_verify_step(pool.handle, [0], [3], 2, 256, 256, 256, 256, 256, 1 << 20, None)
    assert before == (pool.stats(), pool.block_table(0).tolist())


def _compare(pool, ref):
    ids = sorted(ref.tables)
    assert pool.sequences().tolist() == ids
    for s in ids:
        assert pool.block_table(s).tolist() == ref.tables[s]
        assert pool.seq_len(s) == ref.lengths[s]
    assert [pool.refcount(b) for b in range(ref.num_blocks)] == ref.refs.tolist()
    assert pool.stats() == ref.stats()
    assert pool.pending_copies() == ref.copies


@pytest.mark.parametrize("seed", range(6))
def test_differential_fuzz_against_oracle(seed):
    rng = np.random.default_rng(1000 + seed)
    n_blocks = int(rng.integers(4, 40))
    bs = int(rng.choice([1, 2, 3, 4, 16]))
    order = rng.permutation(n_blocks).tolist()
    ref = Pool(n_blocks, bs, allocation_order=order, store_values=False)
    pool = _meta(n_blocks, bs, order=order)
    live, next_id = [], 0
    for step in range(300):
        kind = int(rng.integers(0, 7))
        if kind == 0 or not live:
            seq = next_id if rng.random() < 0.9 or not live else live[0]
            next_id += 1
            calls = [(ref.create, (seq,)), (pool.create, (seq,))]
        elif kind in (1, 2, 3):
            seq = live[int(rng.integers(len(live)))] if rng.random() < 0.95 else -7
            n = int(rng.integers(0, 3 * bs + 2))
            calls = [(ref.append, (seq, n)), (pool.append, (seq, n))]
        elif kind == 4:
            src = live[int(rng.integers(len(live)))]
            prefix = int(rng.integers(0, ref.lengths[src] + 2))
            dst = next_id if rng.random() < 0.9 else src
            next_id += 1
            calls = [(ref.share, (src, dst, prefix)), (pool.share, (src, dst, prefix))]
        elif kind == 5:
            src = live[int(rng.integers(len(live)))]
            dst = next_id
            next_id += 1
            calls = [(ref.fork, (src, dst)), (pool.fork, (src, dst))]
        else:
            seq = live[int(rng.integers(len(live)))] if rng.random() < 0.95 else -3
            calls = [(ref.release, (seq,)), (pool.release, (seq,))]
        results = []
        for fn, args in calls:
            try:
                results.append(("ok", fn(*args)))
            except MemoryError:
                results.append(("oom", None))
            except KeyError:
                results.append(("unknown", None))
            except ValueError:
                results.append(("invalid", None))
        (r_kind, r_val), (p_kind, p_val) = results
        assert r_kind == p_kind, (step, calls[0][0].__name__, results)
        if r_kind == "ok" and r_val is not None:
            assert list(p_val) == list(r_val)
        live = sorted(ref.tables)
        _compare(pool, ref)
        ref.validate()
        pool.validate()


@pytest.mark.parametrize("seed", range(4))
def test_append_batch_is_sequential_appends_or_nothing(seed):
    rng = np.random.default_rng(77 + seed)
    n_blocks, bs = int(rng.integers(6, 30)), int(rng.choice([1, 2, 4]))
    order = rng.permutation(n_blocks).tolist()
    ref = Pool(n_blocks, bs, allocation_order=order, store_values=False)
    pool = _meta(n_blocks, bs, order=order)
    for s in range(4):
        ref.create(s)
        pool.create(s)
    ref.append(0, 3)
    pool.append(0, 3)
    ref.fork(0, 4)
    pool.fork(0, 4)
    for step in range(40):
        seqs = [int(x) for x in rng.choice([0, 1, 2, 3, 4], size=int(rng.integers(1, 6)))]
        ns = [int(x) for x in rng.integers(0, 2 * bs + 1, size=len(seqs))]
        snapshot = (ref.snapshot(), list(ref.copies), ref.refs.copy(), sorted(ref.free))
        want = []
        try:
            for s, n in zip(seqs, ns):
                want += ref.append(s, n)
            ok = True
        except MemoryError:
            ok = False
        if ok:
            got = pool.append_batch(seqs, ns)
            assert got.tolist() == want
        else:
            # Restore the oracle to the state before the batch.
            ref = Pool(n_blocks, bs, allocation_order=order, store_values=False)
            pool_state = snapshot
            with pytest.raises(OutOfBlocksError):
                pool.append_batch(seqs, ns)
            assert pool.stats() == {k: v for k, v in pool_state[0].items() if k != "sequences"}
            assert pool.pending_copies() == pool_state[1]
            assert [pool.refcount(b) for b in range(n_blocks)] == pool_state[2].tolist()
            for name, entry in pool_state[0]["sequences"].items():
                assert pool.block_table(int(name)).tolist() == entry["blocks"]
                assert pool.seq_len(int(name)) == entry["length"]
            pool.validate()
            return
        _compare(pool, ref)
        pool.validate()


def test_timing_samples_without_launches():
    """No launch was timed since the reset: no samples and a zero total;
    bad kernel ids and counts are rejected (host only, no GPU call)."""
    abi.pa_timing_reset()
    assert abi.pa_timing_samples(abi.PA_KERNEL_DECODE) == []
    assert abi.pa_timing_read(abi.PA_KERNEL_DECODE) == (0.0, 0)
    lib = abi.load()
    n = abi._i64()
    assert lib.pa_timing_samples(abi.PA_KERNEL_COUNT, None, 0, abi.ctypes.byref(n)) != 0
    assert lib.pa_timing_samples(0, None, -1, abi.ctypes.byref(n)) != 0
    assert lib.pa_timing_samples(0, None, 4, abi.ctypes.byref(n)) != 0
    assert lib.pa_timing_samples(0, None, 0, None) != 0
