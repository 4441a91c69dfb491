"""Pool model of the oracle: physical blocks, refcounts, block tables, COW.

Test infrastructure only (see the package docstring).

The model follows two pages:

* abhik.ai "examples/pagedattention.py", class ``KVPool``: a fixed pool of
  physical blocks, an authored ``allocation_order`` (a full permutation of the
  block ids), refcounts, per-sequence block tables and lengths; a new block is
  the first free id in that order (region physical_pool and ``_allocate``);
  a token position maps to ``(table[p // block_size], p % block_size)``
  (region logical_address); appending into a shared, partially filled tail
  first copies that whole block to a fresh one (region copy_on_write); fork
  copies the parent's table and bumps every refcount (region fork_prefix);
  release drops refcounts and frees blocks that reach zero (region
  release_sequence).
* vladkulikov.com notebook "Модуль 10", class ``PagedKVPool``: multi-token
  append with a preflight block count (one extra block when the tail is
  partial and shared, plus whole blocks for what does not fit in the tail),
  checked before anything changes; ``share_prefix`` giving the target the
  first ``ceil(prefix / block_size)`` blocks; the fill / payload / waste /
  savings accounting; and the ``validate`` invariants.

Where the two pages differ, the readings are:

* next free block: the smallest rank in ``allocation_order`` (the first
  page's rule); the second page's free list is a LIFO stack, which gives the
  same ids on every trace either page prints, since none allocates after a
  release;
* a copy-on-write copies the whole block (first page); only live slots are
  ever read;
* ``fork(src, dst)`` is ``share(src, dst, len(src))``; the first page's
  context tuple is not modelled (one pool per model and layer).

Pins: a block can also be referenced from outside every block table (the
prefix cache of :mod:`oracle.prefix` holds one reference per cached block).
Such a reference counts in the refcount, so the block stays allocated after
every sequence holding it is released; a block only pins hold has fill 0 (no
live sequence uses its slots), so it counts as capacity, not payload.

Windows: a sequence can carry a (sinks, recent) window (oracle.window).  An
append then releases the pages that lie wholly between the sink pages and
the window of its first appended row; such a table entry becomes ``HOLE``
(its position stays counted in the length).  A rollback (``truncate``) may
not fall before the resident window.

Storage: ``K`` and ``V`` are float64 arrays ``[num_blocks, block_size,
num_kv_heads, head_dim]`` -- block, slot, head, dim -- the first page's
``keys[num_blocks, block_size, dim]`` with a KV-head axis added in the
``[kv_len, num_kv_heads, head_dim]`` token order of ferrum-kv's
``paged_attention``.  The oracle copies a block at the moment of the COW; it
also records the ``(src, dst)`` pair so a test can compare the list of copies
a device implementation must perform.
"""

from __future__ import annotations

import heapq
import math

import numpy as np

from .fp8 import dequantize_rows_fp8, quantize_rows_fp8
from .quant import code_limit, dequantize_rows, quantize_rows, stored_scale


class OutOfBlocks(MemoryError):
    """The preflight found fewer free blocks than the operation needs."""


class UnknownSequence(KeyError):
    """The sequence id is not live (never created, or already released)."""


class SequenceExists(ValueError):
    """The sequence id is already live."""


def _positive_int(value, name):
    if isinstance(value, bool) or not isinstance(value, (int, np.integer)) or value <= 0:
        raise ValueError(f"{name} must be a positive integer")
    return int(value)


def _non_negative_int(value, name):
    if isinstance(value, bool) or not isinstance(value, (int, np.integer)) or value < 0:
        raise ValueError(f"{name} must be a non-negative integer")
    return int(value)


def _ceil_div(a, b):
    return -(-a // b)


HOLE = -1  # table entry of a page released by the window policy


class Pool:
    """Fixed pool of physical KV blocks shared by refcounted block tables."""

    def __init__(self, num_blocks, block_size, num_kv_heads=1, head_dim=1,
                 allocation_order=None, store_values=True, quant_bits=None, quant_fp8=False):
        self.num_blocks = _positive_int(num_blocks, "num_blocks")
        self.block_size = _positive_int(block_size, "block_size")
        self.num_kv_heads = _positive_int(num_kv_heads, "num_kv_heads")
        self.head_dim = _positive_int(head_dim, "head_dim")
        if allocation_order is None:
            order = list(range(self.num_blocks))
        else:
            order = [int(x) for x in allocation_order]
        if sorted(order) != list(range(self.num_blocks)):
            raise ValueError("allocation_order must be a full permutation")
        self.order = tuple(order)
        # rank[b] = position of block b in the authored order.
        self.rank = [0] * self.num_blocks
        for position, block in enumerate(self.order):
            self.rank[block] = position
        self.refs = np.zeros(self.num_blocks, dtype=np.int64)
        # References held outside the block tables (the prefix cache's).
        self.pins = np.zeros(self.num_blocks, dtype=np.int64)
        self.free = set(range(self.num_blocks))
        # Free blocks keyed by rank; heap pop = first free id in the order.
        self._free_heap = [(self.rank[b], b) for b in range(self.num_blocks)]
        heapq.heapify(self._free_heap)
        self.tables: dict[int, list[int]] = {}
        self.lengths: dict[int, int] = {}
        # Window policy (sinks, recent) of windowed sequences (oracle.window);
        # an evicted page's table entry is HOLE.
        self.windows: dict = {}
        self.copies: list[tuple[int, int]] = []
        self.store_values = bool(store_values)
        if self.store_values:
            shape = (self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim)
            self.K = np.zeros(shape, dtype=np.float64)
            self.V = np.zeros(shape, dtype=np.float64)
        # Quantised storage (oracle.quant; with quant_fp8, oracle.fp8's 8-bit
        # float codes): codes and the fp32 scale of every (slot, head) row;
        # K / V then hold the values read back.
        self.quant_bits = None
        self.quant_fp8 = bool(quant_fp8)
        if self.quant_fp8 and quant_bits is None:
            quant_bits = 8
        if self.quant_fp8 and quant_bits != 8:
            raise ValueError("8-bit float codes have 8 bits")
        if quant_bits is not None:
            if not self.store_values:
                raise ValueError("quant_bits needs store_values")
            self.quant_bits = int(quant_bits)
            code_limit(self.quant_bits)
            self.Kc = np.zeros(shape, dtype=np.int64)
            self.Vc = np.zeros(shape, dtype=np.int64)
            self.Ks = np.ones(shape[:3], dtype=np.float64)
            self.Vs = np.ones(shape[:3], dtype=np.float64)

    # ------------------------------------------------------------ lookups
    def _existing(self, seq):
        if seq not in self.tables:
            raise UnknownSequence(seq)
        return seq

    def _new(self, seq):
        if seq in self.tables:
            raise SequenceExists(seq)
        return seq

    def sequence_length(self, seq):
        return self.lengths[self._existing(seq)]

    def page_table(self, seq):
        return tuple(self.tables[self._existing(seq)])

    # ------------------------------------------------------------ allocation
    def _allocate(self):
        """First free block in the authored allocation order; refcount 1."""
        if not self.free:
            raise OutOfBlocks("physical KV pool exhausted")
        while True:
            _, block = heapq.heappop(self._free_heap)
            if block in self.free:
                break
        self.free.remove(block)
        self.refs[block] = 1
        return block

    def _drop_ref(self, block):
        self.refs[block] -= 1
        if self.refs[block] == 0:
            self.free.add(block)
            heapq.heappush(self._free_heap, (self.rank[block], block))

    # ------------------------------------------------------------ operations
    def create(self, seq):
        """Empty table, length 0; nothing is reserved up front."""
        self._new(seq)
        self.tables[seq] = []
        self.lengths[seq] = 0

    def blocks_needed(self, seq, n):
        """Preflight count for appending ``n`` tokens to ``seq``."""
        length = self.lengths[self._existing(seq)]
        if n == 0:
            return 0
        need = 0
        remainder = length % self.block_size
        room = 0
        if remainder:
            if self.refs[self.tables[seq][-1]] > 1:
                need += 1  # copy-on-write replacement of the shared tail
            room = self.block_size - remainder
        need += _ceil_div(max(0, n - room), self.block_size)
        return need

    def append(self, seq, n):
        """Append ``n`` logical tokens; return the slot of each new position.

        Preflight first: if the pool cannot supply every block the append
        needs, raise :class:`OutOfBlocks` and change nothing.  Then a shared
        partial tail is replaced by a private copy, the tail is filled and
        whole new blocks are taken in allocation order.
        """
        n = _non_negative_int(n, "n_tokens")
        self._existing(seq)
        need = self.blocks_needed(seq, n)
        if need > len(self.free):
            raise OutOfBlocks(f"need {need} free blocks, {len(self.free)} remain")
        table = self.tables[seq]
        length = self.lengths[seq]
        if n and length % self.block_size:
            old = table[-1]
            if self.refs[old] > 1:
                new = self._allocate()
                if self.store_values:
                    self.K[new] = self.K[old]
                    self.V[new] = self.V[old]
                if self.quant_bits is not None:
                    for arr in (self.Kc, self.Vc, self.Ks, self.Vs):
                        arr[new] = arr[old]
                self.copies.append((old, new))
                table[-1] = new
                self._drop_ref(old)
        first = length
        for _ in range(_ceil_div(length + n, self.block_size) - len(table)):
            table.append(self._allocate())
        self.lengths[seq] = length + n
        slots = [self.slot(seq, p) for p in range(first, first + n)]
        if n and seq in self.windows:
            self._evict(seq, first)
        return slots

    # ------------------------------------------------------------ windows
    def set_window(self, seq, sinks, recent):
        """Give ``seq`` a (sinks, recent) window: its queries see the
        positions oracle.window.window_keep keeps, and appends release the pages no later query of
        the appended rows can see."""
        self._existing(seq)
        sinks = _non_negative_int(sinks, "sinks")
        recent = _non_negative_int(recent, "recent")
        if sinks + recent < 1:
            raise ValueError("the window must keep at least one token")
        self.windows[seq] = (sinks, recent)

    def _evict(self, seq, first_new):
        """Release the pages that lie wholly after the sink pages and before
        the window of the first appended row (position ``first_new``, which
        sees ``[first_new + 1 - recent, first_new]``); pages holding appended
        rows are kept."""
        sinks, recent = self.windows[seq]
        bs = self.block_size
        table = self.tables[seq]
        sink_pages = _ceil_div(sinks, bs)
        lo = first_new + 1 - recent
        end = min(max(lo, 0) // bs, first_new // bs)
        for j in range(sink_pages, end):
            if table[j] != HOLE:
                self._drop_ref(table[j])
                table[j] = HOLE

    def evicted_end(self, seq):
        """Position where the resident part after the sinks starts (0 when
        nothing was released)."""
        table = self.tables[self._existing(seq)]
        last = max((j for j, b in enumerate(table) if b == HOLE), default=-1)
        return (last + 1) * self.block_size if last >= 0 else 0

    def truncate(self, seq, new_length):
        """Drop the positions from ``new_length`` on (a rollback).  Evicted
        positions cannot come back: ``new_length`` must not fall before the
        resident window."""
        self._existing(seq)
        new_length = _non_negative_int(new_length, "new_length")
        length = self.lengths[seq]
        if new_length > length:
            raise ValueError("new_length exceeds the sequence length")
        if new_length < self.evicted_end(seq):
            raise ValueError("rollback lies outside the retained interval")
        table = self.tables[seq]
        keep = _ceil_div(new_length, self.block_size)
        for block in table[keep:]:
            if block != HOLE:
                self._drop_ref(block)
        del table[keep:]
        self.lengths[seq] = new_length

    def resident(self, seq):
        """(positions, K, V) of the resident positions of ``seq``, ascending."""
        length = self.lengths[self._existing(seq)]
        table = self.tables[seq]
        pos = [p for p in range(length) if table[p // self.block_size] != HOLE]
        keys = np.empty((len(pos), self.num_kv_heads, self.head_dim))
        values = np.empty_like(keys)
        for i, p in enumerate(pos):
            block, offset = table[p // self.block_size], p % self.block_size
            keys[i] = self.K[block, offset]
            values[i] = self.V[block, offset]
        return pos, keys, values

    def share(self, src, dst, prefix):
        """New sequence ``dst`` holding the blocks covering ``src[:prefix]``
        (a windowed source's released pages included; the prefix may not end
        before its resident window)."""
        self._existing(src)
        prefix = _non_negative_int(prefix, "prefix_tokens")
        if prefix > self.lengths[src]:
            raise ValueError("prefix_tokens exceeds source length")
        if prefix < self.evicted_end(src):
            raise ValueError("the prefix ends among released positions")
        self._new(dst)
        table = self.tables[src][:_ceil_div(prefix, self.block_size)]
        for block in table:
            if block != HOLE:
                self.refs[block] += 1
        self.tables[dst] = list(table)
        self.lengths[dst] = prefix
        if src in self.windows:
            self.windows[dst] = self.windows[src]

    def fork(self, src, dst):
        """Child with the parent's whole table (every refcount + 1)."""
        self._existing(src)
        self.share(src, dst, self.lengths[src])

    def adopt(self, seq, blocks, length):
        """New sequence ``seq`` whose table is ``blocks`` (each refcount + 1)
        and whose length is ``length``; ``ceil(length / block_size)`` must be
        ``len(blocks)`` and every block must be referenced already."""
        self._new(seq)
        length = _non_negative_int(length, "length")
        blocks = [int(b) for b in blocks]
        if _ceil_div(length, self.block_size) != len(blocks) or len(set(blocks)) != len(blocks):
            raise ValueError("blocks must cover length exactly, each once")
        if any(not 0 <= b < self.num_blocks or self.refs[b] == 0 for b in blocks):
            raise ValueError("adopted blocks must be live")
        for b in blocks:
            self.refs[b] += 1
        self.tables[seq] = blocks
        self.lengths[seq] = length

    def pin(self, block):
        """One more reference to a live block, held outside every table."""
        if self.refs[block] == 0:
            raise ValueError("only a live block can be pinned")
        self.refs[block] += 1
        self.pins[block] += 1

    def unpin(self, block):
        if self.pins[block] == 0:
            raise ValueError("block is not pinned")
        self.pins[block] -= 1
        self._drop_ref(block)

    def release(self, seq):
        """Drop one reference per block; blocks at zero become free."""
        self._existing(seq)
        for block in self.tables[seq]:
            if block != HOLE:
                self._drop_ref(block)
        del self.tables[seq]
        del self.lengths[seq]
        self.windows.pop(seq, None)

    # ------------------------------------------------------------ addressing
    def address(self, seq, p):
        """(physical block, offset) of live token position ``p``."""
        self._existing(seq)
        if not 0 <= p < self.lengths[seq]:
            raise ValueError("token index must address a live token")
        logical, offset = divmod(p, self.block_size)
        if self.tables[seq][logical] == HOLE:
            raise ValueError("token index addresses an evicted page")
        return self.tables[seq][logical], offset

    def slot(self, seq, p):
        block, offset = self.address(seq, p)
        return block * self.block_size + offset

    def write(self, slots, k, v):
        """Store rows ``k[i], v[i]`` (each ``[num_kv_heads, head_dim]``) at slots.

        A quantised pool stores the codes and fp32 scales of each head's row
        and keeps the values they read back as K / V."""
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        for i, slot in enumerate(slots):
            block, offset = divmod(int(slot), self.block_size)
            if self.quant_bits is None:
                self.K[block, offset] = k[i]
                self.V[block, offset] = v[i]
                continue
            for rows, codes_arr, scale_arr, vals in ((k[i], self.Kc, self.Ks, self.K),
                                                     (v[i], self.Vc, self.Vs, self.V)):
                if self.quant_fp8:
                    codes, scale = quantize_rows_fp8(rows)
                    scale = stored_scale(scale)
                    vals[block, offset] = dequantize_rows_fp8(codes, scale)
                else:
                    codes, scale = quantize_rows(rows, self.quant_bits)
                    scale = stored_scale(scale)
                    vals[block, offset] = dequantize_rows(codes, scale)
                codes_arr[block, offset] = codes
                scale_arr[block, offset] = scale[:, 0]

    def gather(self, seq):
        """Live K/V rows in logical order: two arrays ``[len, Hkv, D]``."""
        length = self.lengths[self._existing(seq)]
        keys = np.empty((length, self.num_kv_heads, self.head_dim))
        values = np.empty((length, self.num_kv_heads, self.head_dim))
        for p in range(length):
            block, offset = self.address(seq, p)
            keys[p] = self.K[block, offset]
            values[p] = self.V[block, offset]
        return keys, values

    # ------------------------------------------------------------ accounting
    def fills(self):
        """Per block: the largest number of live slots any owner uses."""
        fill = [0] * self.num_blocks
        for seq, table in self.tables.items():
            length = self.lengths[seq]
            for j, block in enumerate(table):
                if block != HOLE:
                    fill[block] = max(fill[block], min(self.block_size, length - j * self.block_size))
        return fill

    def stats(self):
        allocated = self.num_blocks - len(self.free)
        capacity = allocated * self.block_size
        payload = sum(f for b, f in enumerate(self.fills()) if self.refs[b])
        logical = sum(self.lengths.values())
        return {
            "allocated_blocks": allocated,
            "free_blocks": len(self.free),
            "physical_capacity_tokens": capacity,
            "physical_payload_tokens": payload,
            "logical_tokens": logical,
            "internal_waste_tokens": capacity - payload,
            "sharing_savings_tokens": logical - payload,
        }

    def snapshot(self, names=None):
        """Stats plus ``{name: {"blocks", "length"}}`` for every live sequence."""
        out = dict(self.stats())
        out["sequences"] = {
            (names[s] if names else str(s)): {"blocks": list(t), "length": self.lengths[s]}
            for s, t in sorted(self.tables.items(), key=lambda item: repr(item[0]))
        }
        return out

    def validate(self):
        """Invariants of the second page's ``validate``; AssertionError if broken."""
        expected = [0] * self.num_blocks
        for seq, table in self.tables.items():
            length = self.lengths[seq]
            assert length >= 0, "negative length"
            assert len(table) == _ceil_div(length, self.block_size), "table length"
            live = [b for b in table if b != HOLE]
            assert len(set(live)) == len(live), "block twice in one table"
            if table and length % self.block_size:
                assert table[-1] != HOLE, "a partially filled tail page is evicted"
            for block in live:
                assert 0 <= block < self.num_blocks, "block id out of range"
                expected[block] += 1
        fill = self.fills()
        for block in range(self.num_blocks):
            assert self.refs[block] == expected[block] + self.pins[block], \
                "refcount != table references + pins"
            if self.refs[block] == 0:
                assert block in self.free and fill[block] == 0, "unreferenced block not free"
            elif expected[block] == 0:
                assert block not in self.free and fill[block] == 0, "pinned-only block"
            else:
                assert block not in self.free, "referenced block is free"
                assert 1 <= fill[block] <= self.block_size, "fill out of range"
        stats = self.stats()
        assert stats["logical_tokens"] >= stats["physical_payload_tokens"], "payload > logical"
