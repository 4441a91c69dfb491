"""GPU parity of sliding-window attention with sinks at page granularity:
decode, the verify step and prefill over windowed sequences whose released
pages are gone, against the oracle's windowed attention over the resident
rows.

Source: vladkulikov.com notebook "Модуль 10", eviction cell
(streaming_keep_indices) and explicit window caches.  Bar: tables and
refcounts bit-exact; outputs within (2e-3, 1e-2) of the float64 oracle
((1e-5, 1e-5) for the fp32 pool).
"""

import numpy as np
import pytest

import oracle
from oracle.pool import HOLE
from synth.workloads import bf16_round, to_f64

from gpu_support import BF16_TOL, F32_TOL, assert_close, log, to_device, to_host_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_block_amd import abi
    abi.load()


def _draw(rng, shape, dtype):
    x = rng.standard_normal(shape).astype(np.float32)
    return bf16_round(x) if dtype != "f32" else x


def _io(dtype):
    return "f32" if dtype == "f32" else "bf16"


def _build(specs, hq, hkv, d, bs, kv, chunk=64, seed=3):
    """specs: [(length, window or None)], each sequence appended in chunks
    of ``chunk`` tokens with its K/V written after every append."""
    from paged_kv_cache_block_amd import DevicePool
    nb = int(sum(-(-n // bs) + 2 for n, _ in specs) + 32)
    order = np.random.default_rng(seed).permutation(nb).astype(np.int32)
    pool = DevicePool(nb, bs, hkv, d, dtype=kv, allocation_order=order)
    ref = oracle.Pool(nb, bs, hkv, d, allocation_order=order, quant_bits=8 if kv in ("i8", "fp8") else None,
                     quant_fp8=kv == "fp8")
    rng = np.random.default_rng(seed + 1)
    io = _io(kv)
    for s, (n, win) in enumerate(specs):
        pool.create(s)
        ref.create(s)
        if win is not None:
            pool.set_window(s, *win)
            ref.set_window(s, *win)
        done = 0
        while done < n:
            m = min(chunk, n - done)
            k, v = _draw(rng, (m, hkv, d), kv), _draw(rng, (m, hkv, d), kv)
            slots = pool.append(s, m)
            assert slots.tolist() == ref.append(s, m)
            pool.write(slots, to_device(k, io), to_device(v, io))
            ref.write(slots, to_f64(k, io), to_f64(v, io))
            done += m
    torch.cuda.synchronize()
    return pool, ref, rng


def _want(ref, s, q_rows, io):
    pos, keys, values = ref.resident(s)
    win = ref.windows.get(s)
    L = ref.lengths[s]
    if win is None:
        return oracle.attention(to_f64(q_rows, io), keys, values)
    return oracle.windowed_attention(to_f64(q_rows, io), keys, values, pos, L, *win)


def _check_tables(pool, ref, seqs):
    for s in seqs:
        assert pool.block_table(s).tolist() == ref.tables[s]
    assert [pool.refcount(b) for b in range(ref.num_blocks)] == ref.refs.tolist()


WINDOW_SPECS = [
    (5000, (4, 1000)),     # sinks + window, split-K over the visited pages
    (3000, (0, 512)),      # plain sliding window
    (700, (16, 200)),      # sinks on a page boundary
    (2100, (5, 0)),        # sinks only (recent 0)
    (90, (4, 500)),        # shorter than the budget: sees everything
    (1500, None),          # no window, in the same batch
]


@pytest.mark.parametrize("kv,hq,hkv,d,bs", [("bf16", 32, 8, 128, 16), ("i8", 32, 8, 128, 16),
                                            ("fp8", 32, 8, 128, 16), ("bf16", 16, 16, 64, 32)],
                         ids=["bf16-G4", "i8-G4", "fp8-G4", "bf16-MHA-bs32"])
def test_windowed_decode(kv, hq, hkv, d, bs):
    log(f"windowed decode {kv}")
    pool, ref, rng = _build(WINDOW_SPECS, hq, hkv, d, bs, kv)
    seqs = list(range(len(WINDOW_SPECS)))
    _check_tables(pool, ref, seqs)
    assert HOLE in ref.tables[0] and HOLE in ref.tables[1]
    q = _draw(rng, (len(seqs), hq, d), "bf16")
    got = to_host_f64(pool.decode(seqs, to_device(q, "bf16")))
    for i, s in enumerate(seqs):
        assert_close(got[i], _want(ref, s, q[i:i + 1], "bf16")[0], *BF16_TOL, what=f"seq {s} {WINDOW_SPECS[s]}")


@pytest.mark.parametrize("kv", ["bf16", "i8", "fp8"])
def test_windowed_decode_and_verify_steps_with_rollback(kv):
    hq, hkv, d, bs = 32, 8, 128, 16
    specs = [(1200, (4, 300)), (600, (0, 100)), (2000, None)]
    pool, ref, rng = _build(specs, hq, hkv, d, bs, kv)
    seqs = [0, 1, 2]
    for step in range(6):
        if step % 2 == 0:
            q_lens = [1, 1, 1]
        else:
            q_lens = [4, 8, 2]
        R = sum(q_lens)
        k, v, q = _draw(rng, (R, hkv, d), "bf16"), _draw(rng, (R, hkv, d), "bf16"), _draw(rng, (R, hq, d), "bf16")
        if step % 2 == 0:
            out, slots = pool.decode_step(seqs, to_device(k, "bf16"), to_device(v, "bf16"), to_device(q, "bf16"))
        else:
            out, slots = pool.verify_step(seqs, q_lens, to_device(k, "bf16"), to_device(v, "bf16"), to_device(q, "bf16"))
        want_slots = []
        for s, n in zip(seqs, q_lens):
            want_slots += ref.append(s, n)
        assert slots.tolist() == want_slots
        ref.write(want_slots, to_f64(k, "bf16"), to_f64(v, "bf16"))
        got = to_host_f64(out)
        r0 = 0
        for s, n in zip(seqs, q_lens):
            assert_close(got[r0:r0 + n], _want(ref, s, q[r0:r0 + n], "bf16"), *BF16_TOL, what=f"step {step} seq {s}")
            r0 += n
        if step % 2 == 1:
            # Reject all but the first two verified tokens of each sequence.
            for s, n in zip(seqs, q_lens):
                keep = ref.lengths[s] - n + min(n, 2)
                pool.truncate(s, keep)
                ref.truncate(s, keep)
        _check_tables(pool, ref, seqs)
    pool.validate()


def test_windowed_prefill_long_chunk_and_fp32_generic():
    hq, hkv, d, bs = 32, 8, 128, 16
    specs = [(900, (4, 128)), (400, None)]
    pool, ref, rng = _build(specs, hq, hkv, d, bs, "bf16", chunk=300)
    q_lens = [300, 100]   # the last chunk of sequence 0 and 100 rows of sequence 1
    q = _draw(rng, (sum(q_lens), hq, d), "bf16")
    got = to_host_f64(pool.prefill([0, 1], q_lens, to_device(q, "bf16")))
    assert_close(got[:300], _want(ref, 0, q[:300], "bf16"), *BF16_TOL, what="windowed prefill")
    assert_close(got[300:], _want(ref, 1, q[300:], "bf16"), *BF16_TOL, what="plain prefill")
    # fp32 pool: the generic kernel.
    pool32, ref32, rng = _build([(333, (3, 50)), (120, (0, 7))], 8, 2, 32, 8, "f32", chunk=40)
    q32 = _draw(rng, (2, 8, 32), "f32")
    got = to_host_f64(pool32.decode([0, 1], to_device(q32, "f32")))
    for s in range(2):
        assert_close(got[s], _want(ref32, s, q32[s:s + 1], "f32")[0], *F32_TOL, what=f"fp32 seq {s}")


@pytest.mark.parametrize("kv", ["bf16", "i8"])
def test_balanced_windowed_batch_runs_unsplit(kv):
    """32 windowed rows of equal visited length over 8 KV heads (256
    workgroups): the work list leaves every row whole (one range, no split-K
    partials, no merge launch), and the outputs still match the oracle."""
    log(f"balanced windowed batch {kv}")
    specs = [(1100 + 3 * i, (4, 1024)) for i in range(32)]
    pool, ref, rng = _build(specs, 32, 8, 128, 16, kv, chunk=256)
    seqs = list(range(len(specs)))
    _, items, _ = pool.decode_work_items(seqs, 32)
    assert len(items) == len(seqs) and (items[:, 10] == -1).all()
    q = _draw(rng, (len(seqs), 32, 128), "bf16")
    got = to_host_f64(pool.decode(seqs, to_device(q, "bf16")))
    for i, s in enumerate(seqs):
        assert_close(got[i], _want(ref, s, q[i:i + 1], "bf16")[0], *BF16_TOL, what=f"seq {s}")
    k, v = _draw(rng, (len(seqs), 8, 128), "bf16"), _draw(rng, (len(seqs), 8, 128), "bf16")
    q = _draw(rng, (len(seqs), 32, 128), "bf16")
    out, slots = pool.decode_step(seqs, to_device(k, "bf16"), to_device(v, "bf16"), to_device(q, "bf16"))
    want_slots = []
    for s in seqs:
        want_slots += ref.append(s, 1)
    assert slots.tolist() == want_slots
    ref.write(want_slots, to_f64(k, "bf16"), to_f64(v, "bf16"))
    got = to_host_f64(out)
    for i, s in enumerate(seqs):
        assert_close(got[i], _want(ref, s, q[i:i + 1], "bf16")[0], *BF16_TOL, what=f"step seq {s}")
    _check_tables(pool, ref, seqs)


PREFILL_SPECS = [
    # (length, window, wanted rows): the rows are capped at the positions
    # still resident, so early rows of a long chunk may find pages of their
    # own window already released (their keys are gone).
    (1500, (4, 256), 400),
    (3000, (0, 512), 200),
    (700, (40, 100), 150),    # sinks over two key tiles
    (2100, (5, 0), 50),       # sinks only
    (90, (4, 500), 90),       # shorter than the budget; rows reach position 0
    (1500, None, 256),        # no window, in the same call
]


@pytest.mark.parametrize("kv,hq,hkv,d,bs", [("bf16", 32, 8, 128, 16), ("i8", 32, 8, 128, 16),
                                            ("bf16", 16, 16, 64, 32), ("i8", 16, 8, 64, 32),
                                            ("fp8", 32, 8, 128, 16), ("fp8", 16, 8, 64, 32)],
                         ids=["bf16-G4-D128", "i8-G4-D128", "bf16-MHA-D64-bs32", "i8-G2-D64-bs32",
                              "fp8-G4-D128", "fp8-G2-D64-bs32"])
def test_windowed_prefill_mfma(kv, hq, hkv, d, bs):
    """Chunked prefill over windowed sequences on the MFMA kernel: sink
    tiles, then the tiles of the rows' windows; released pages are masked."""
    log(f"windowed prefill {kv} G{hq // hkv} D{d} bs{bs}")
    specs = [(n, w) for n, w, _ in PREFILL_SPECS]
    pool, ref, rng = _build(specs, hq, hkv, d, bs, kv)
    seqs = list(range(len(specs)))
    q_lens = [min(want, ref.lengths[s] - ref.evicted_end(s)) for s, (_, _, want) in enumerate(PREFILL_SPECS)]
    assert all(n >= 1 for n in q_lens) and q_lens[0] < PREFILL_SPECS[0][2]
    q = _draw(rng, (sum(q_lens), hq, d), "bf16")
    got = to_host_f64(pool.prefill(seqs, q_lens, to_device(q, "bf16")))
    r0 = 0
    for s, n in zip(seqs, q_lens):
        assert_close(got[r0:r0 + n], _want(ref, s, q[r0:r0 + n], "bf16"), *BF16_TOL,
                     what=f"seq {s} {PREFILL_SPECS[s]} rows {n}")
        r0 += n
