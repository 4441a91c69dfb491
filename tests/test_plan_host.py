"""The decode work list through the C ABI (pa_decode_work_items, host only,
on metadata-only pools) against the oracle pool.

The work list splits docs.rs ferrum-kv 0.4.0 src/attention.rs
paged_attention's key loop into page ranges whose partial results CMU
11-667 lecture 19 section 3 online_softmax_stats merges; what it must get
right is which keys each range reads.  Bar, for random pools (windows with
sinks, released pages, shared prefixes, forks, rollbacks) and batches
(duplicates, multi-row queries): every visited page of a batch row lies in
exactly one of its ranges; the visited pages hold every resident key any
of its query rows sees (oracle.window_keep; vladkulikov.com notebook
"Модуль 10", eviction cell) and no released page; the tables the work list
carries are the pool's tables over those pages, bit-exact; each item
carries its row's length, query rows and window; split rows own disjoint
partial rows; full ranges run before shorter ones, longest first.
"""

import numpy as np
import pytest

import oracle
from oracle.pool import HOLE
from oracle.window import window_keep
from paged_kv_cache_block_amd import DevicePool
from paged_kv_cache_block_amd.abi import InvalidArgumentError, UnknownSequenceError

NO_WINDOW = 1 << 29


def _check(ref, seqs, num_heads, q_lens, ppr, items, tables):
    bs = ref.block_size
    B = len(seqs)
    ql = list(q_lens) if q_lens is not None else [1] * B
    row0 = np.concatenate([[0], np.cumsum(ql)[:-1]]).astype(int)
    ranges = {b: [] for b in range(B)}
    spans = []
    for it in items.tolist():
        b, c, L, r0, q, sinks, recent, sp, gap, toff, base, zero = it[:12]
        s = seqs[b]
        assert (L, r0, q, zero) == (ref.lengths[s], row0[b], ql[b], 0)
        win = ref.windows.get(s)
        assert (sinks, recent) == (tuple(win) if win is not None else (0, NO_WINDOW))
        nblk = -(-L // bs)
        nvis = nblk - gap
        p0, p1 = c * ppr, min(nvis, (c + 1) * ppr)
        assert 0 <= p0 < p1
        ranges[b].append((c, base, toff, sp, gap, nvis))
        spans.append(p1 - p0)
        for w in range(4):
            assert it[12 + w] == (tables[toff + p0 + w] if p0 + w < p1 else 0)
    part_rows = []
    for b in range(B):
        s, L, q = seqs[b], ref.lengths[seqs[b]], ql[b]
        cs = sorted(r[0] for r in ranges[b])
        (base, toff, sp, gap, nvis), = {r[1:] for r in ranges[b]}
        assert cs == list(range(-(-nvis // ppr)))
        assert (base == -1) == (len(cs) == 1)
        if base >= 0:
            part_rows.append((base, base + len(cs) * q * num_heads))
        nblk = -(-L // bs)
        pages = list(range(sp)) + list(range(sp + gap, nblk))
        assert len(pages) == nvis
        assert tables[toff:toff + nvis].tolist() == [ref.tables[s][p] for p in pages]
        assert HOLE not in tables[toff:toff + nvis].tolist()
        win = ref.windows.get(s)
        for t in range(q):
            lim = L - q + t + 1
            kept = window_keep(lim, *win) if win is not None else range(lim)
            for p in kept:
                if ref.tables[s][p // bs] != HOLE:
                    assert p // bs in pages, (s, t, p)
    part_rows.sort()
    for (_, e0), (s1, _) in zip(part_rows, part_rows[1:]):
        assert e0 <= s1
    full = [n == ppr for n in spans]
    assert full == sorted(full, reverse=True)
    tail = [n for n in spans if n != ppr]
    assert tail == sorted(tail, reverse=True)


def _random_pool(seed):
    rng = np.random.default_rng(seed)
    bs = int(rng.choice([1, 4, 16, 32]))
    hkv = int(rng.choice([1, 2, 8]))
    nb = 4096
    order = rng.permutation(nb).astype(np.int32)
    pool = DevicePool(nb, bs, hkv, 64, metadata_only=True, allocation_order=order)
    ref = oracle.Pool(nb, bs, hkv, 64, allocation_order=order, store_values=False)
    live = []
    for s in range(int(rng.integers(3, 12))):
        pool.create(s)
        ref.create(s)
        if rng.random() < 0.35:
            win = (int(rng.integers(0, 20)), int(rng.integers(1, 600)))
            pool.set_window(s, *win)
            ref.set_window(s, *win)
        n = int(np.exp(rng.uniform(0, np.log(9000))))
        done = 0
        while done < n:
            m = min(n - done, int(rng.integers(1, 700)))
            assert pool.append(s, m).tolist() == ref.append(s, m)
            done += m
        live.append(s)
    nxt = 100
    for _ in range(int(rng.integers(0, 4))):  # shares, forks, rollbacks, releases
        s = live[int(rng.integers(len(live)))]
        op = rng.integers(4)
        if op == 0 and s not in ref.windows:
            prefix = int(rng.integers(1, ref.lengths[s] + 1))
            pool.share(s, nxt, prefix)
            ref.share(s, nxt, prefix)
            live.append(nxt)
            nxt += 1
        elif op == 1:
            pool.fork(s, nxt)
            ref.fork(s, nxt)
            live.append(nxt)
            nxt += 1
        elif op == 2:
            new_len = int(rng.integers(max(ref.evicted_end(s), 1), ref.lengths[s] + 1))
            pool.truncate(s, new_len)
            ref.truncate(s, new_len)
        elif len(live) > 2:
            pool.release(s)
            ref.release(s)
            live.remove(s)
        m = int(rng.integers(1, 40))
        t = live[-1]
        assert pool.append(t, m).tolist() == ref.append(t, m)
    return rng, pool, ref, live, hkv


@pytest.mark.parametrize("seed", range(12))
def test_work_list_covers_the_visible_pages(seed):
    rng, pool, ref, live, hkv = _random_pool(seed)
    for _ in range(4):
        num_heads = hkv * int(rng.choice([1, 2, 4, 8]))
        batch = [live[int(i)] for i in rng.integers(0, len(live), size=int(rng.integers(1, 2 * len(live))))]
        ppr, items, tables = pool.decode_work_items(batch, num_heads)
        _check(ref, batch, num_heads, None, ppr, items, tables)
        rows = list(dict.fromkeys(batch))  # multi-row queries: each sequence once
        q_lens = []
        for s in rows:
            resident = ref.lengths[s] - ref.evicted_end(s)
            q_lens.append(int(rng.integers(1, max(1, min(resident, 40)) + 1)))
        ppr, items, tables = pool.decode_work_items(rows, num_heads, q_lens)
        _check(ref, rows, num_heads, q_lens, ppr, items, tables)


def test_work_list_errors():
    pool = DevicePool(64, 16, 2, 64, metadata_only=True)
    pool.create(0)
    pool.create(1)
    pool.append(0, 40)
    with pytest.raises(UnknownSequenceError):
        pool.decode_work_items([0, 7], 4)
    with pytest.raises(InvalidArgumentError):
        pool.decode_work_items([1], 4)            # empty sequence
    with pytest.raises(InvalidArgumentError):
        pool.decode_work_items([0], 3)            # 3 heads over 2 KV heads
    with pytest.raises(InvalidArgumentError):
        pool.decode_work_items([0], 4, [41])      # more rows than tokens
    ppr, items, tables = pool.decode_work_items([0, 0], 4)
    assert len(items) == 2 and tables.tolist() == pool.block_table(0).tolist() * 2


def test_balanced_batch_that_fills_the_gpu_is_not_split():
    """Rows of about equal visited length whose count times the KV heads
    reaches 256 keep one range each (no split-K partials); a batch just short
    of 256 workgroups, or with one row much longer than the mean, is split."""
    pool = DevicePool(8192, 16, 8, 64, metadata_only=True)
    for s in range(40):
        pool.create(s)
        pool.append(s, 2000 + 7 * s if s < 39 else 2000)
    ppr, items, _ = pool.decode_work_items(list(range(32)), 32)
    assert len(items) == 32 and (items[:, 10] == -1).all() and ppr >= -(-2217 // 16)
    _, items, _ = pool.decode_work_items(list(range(31)), 32)       # 248 workgroups
    assert (items[:, 10] >= 0).any()
    pool.append(39, 6000)                                           # one row 4x the others
    _, items, _ = pool.decode_work_items(list(range(31)) + [39], 32)
    assert (items[:, 10] >= 0).any()
