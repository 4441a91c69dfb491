"""The five paged-attention workloads as seeded recipes.

Recipe (one rule for every workload):

* ``rng = numpy.random.default_rng(seed)`` draws, in this order, the sequence
  lengths (where they are random) and then ``allocation_order =
  rng.permutation(num_blocks)``.
* Sequences are created in index order; each appends its tokens as the op
  list says.  The K/V rows of an append come from that sequence's own
  generator ``default_rng([seed, 1, seq])``: ``standard_normal((n, Hkv, D),
  float32)`` for K, then the same for V, one pair of draws per append, in
  op order.  Shared prefixes carry the source's rows.
* Where a workload has outliers, ``default_rng([seed, 3, seq])`` draws one
  ``random((n, Hkv)) < 0.01`` mask per append; the selected rows of both K
  and V are multiplied by 8 (exact in bf16).
* Queries of sequence ``seq`` come from ``default_rng([seed, 2, seq])``,
  ``standard_normal((q_len, Hq, D), float32)``, one draw per attention call
  on that sequence in the order the workload lists its calls (decode calls
  first, then prefill calls).
* bf16 workloads round every drawn value to bfloat16 with round-to-nearest-
  even; arrays are kept as their 16-bit patterns (``uint16``).  fp32
  workloads keep float32.

Workloads (sizes at their defaults; smaller instances keep the structure):

1. ``tiny_fp32`` -- fp32, 1 head, head_dim 8, block_size 4, 8 blocks in a
   seed-0 permutation; A appends 6, B shares A's 6, B appends 3 (copy-on-
   write of the shared partial tail, then one new block); decode on A and
   B, then a 3-row causal prefill on B.
2. ``gqa_decode`` -- 32 query / 8 KV heads, head_dim 128, bf16, block_size
   16, 32 sequences of length uniform in [1, 8192], 32768-block pool.
3. ``long_decode`` -- 64 query / 8 KV heads, head_dim 128, bf16, block_size
   16, 4 sequences of 131072 tokens filling a 32768-block pool.
4. ``prefix_prefill`` -- 16 sequences share a 4096-token prefix (sequence 0
   appends it; 1..15 share it, refcount 16), then each appends its own 512
   tokens and runs a 512-row causal prefill; 32 / 8 heads, head_dim 128,
   bf16, block_size 16, 1024-block pool.
5. ``heavy_tail`` -- 16 = 16 heads, head_dim 64, bf16, block_size 32, 256
   sequences with lengths ``floor(exp(U(ln 16, ln 32768)))`` clipped to
   [16, 32768], pool sized to 90% occupancy, 1% outlier rows x8.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


# --------------------------------------------------------------- dtype helpers
def bf16_round(x):
    """float32 array -> uint16 bfloat16 bit patterns, round-to-nearest-even:
    the high half of the bits plus the carry out of low half + 0x7FFF + the
    high half's lowest bit (all in uint32, no widening)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    hi = u >> 16
    carry = u & 0xFFFF
    carry += 0x7FFF
    carry += hi & 1
    carry >>= 16
    hi += carry
    return hi.astype(np.uint16)


def bf16_bits_to_f32(bits):
    """uint16 bfloat16 bit patterns -> float32 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def to_f64(arr, dtype):
    """Input array (bf16 bits or float32) widened to float64, exactly."""
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float64)


# --------------------------------------------------------------- workload spec
@dataclass
class Workload:
    name: str
    seed: int
    dtype: str                      # "f32" or "bf16"
    num_blocks: int
    block_size: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    allocation_order: np.ndarray    # int32 permutation of num_blocks
    ops: list                       # ("create", s) | ("append", s, n) | ("share", src, dst, prefix)
    decode_seqs: list = field(default_factory=list)
    prefill: list = field(default_factory=list)   # [(seq, q_len)]
    outliers: bool = False

    @property
    def elt_bytes(self):
        return 2 if self.dtype == "bf16" else 4

    def final_lengths(self):
        """Length of every sequence after the op list (bookkeeping only)."""
        lengths = {}
        for op in self.ops:
            if op[0] == "create":
                lengths[op[1]] = 0
            elif op[0] == "append":
                lengths[op[1]] += op[2]
            elif op[0] == "share":
                lengths[op[2]] = op[3]
        return lengths

    def to_f64(self, arr):
        return to_f64(arr, self.dtype)


def _round(x, dtype):
    return bf16_round(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


# --------------------------------------------------------------- constructors
def tiny_fp32():
    seed = 0
    rng = np.random.default_rng(seed)
    order = rng.permutation(8).astype(np.int32)
    a, b = 0, 1
    ops = [("create", a), ("append", a, 6), ("share", a, b, 6), ("append", b, 3)]
    return Workload("tiny_fp32", seed, "f32", 8, 4, 1, 1, 8, order, ops,
                    decode_seqs=[a, b], prefill=[(b, 3)])


def gqa_decode(batch=32, max_len=8192, num_blocks=32768, num_heads=32, num_kv_heads=8,
               head_dim=128, block_size=16, seed=1):
    rng = np.random.default_rng(seed)
    lengths = rng.integers(1, max_len + 1, size=batch)
    order = rng.permutation(num_blocks).astype(np.int32)
    ops = []
    for i, n in enumerate(lengths):
        ops += [("create", i), ("append", i, int(n))]
    return Workload("gqa_decode", seed, "bf16", num_blocks, block_size, num_heads,
                    num_kv_heads, head_dim, order, ops, decode_seqs=list(range(batch)))


def long_decode(batch=4, length=131072, num_blocks=32768, num_heads=64, num_kv_heads=8,
                head_dim=128, block_size=16, seed=2):
    rng = np.random.default_rng(seed)
    order = rng.permutation(num_blocks).astype(np.int32)
    ops = []
    for i in range(batch):
        ops += [("create", i), ("append", i, length)]
    return Workload("long_decode", seed, "bf16", num_blocks, block_size, num_heads,
                    num_kv_heads, head_dim, order, ops, decode_seqs=list(range(batch)))


def prefix_prefill(batch=16, prefix=4096, chunk=512, num_blocks=1024, num_heads=32,
                   num_kv_heads=8, head_dim=128, block_size=16, seed=3):
    rng = np.random.default_rng(seed)
    order = rng.permutation(num_blocks).astype(np.int32)
    ops = [("create", 0), ("append", 0, prefix)]
    for i in range(1, batch):
        ops.append(("share", 0, i, prefix))
    for i in range(batch):
        ops.append(("append", i, chunk))
    return Workload("prefix_prefill", seed, "bf16", num_blocks, block_size, num_heads,
                    num_kv_heads, head_dim, order, ops,
                    prefill=[(i, chunk) for i in range(batch)])


def heavy_tail(batch=256, min_len=16, max_len=32768, occupancy=0.9, num_heads=16,
               num_kv_heads=16, head_dim=64, block_size=32, seed=4):
    rng = np.random.default_rng(seed)
    lengths = np.floor(np.exp(rng.uniform(math.log(min_len), math.log(max_len), size=batch)))
    lengths = np.clip(lengths.astype(np.int64), min_len, max_len)
    blocks_used = int(sum(-(-int(n) // block_size) for n in lengths))
    num_blocks = math.ceil(blocks_used / occupancy)
    order = rng.permutation(num_blocks).astype(np.int32)
    ops = []
    for i, n in enumerate(lengths):
        ops += [("create", i), ("append", i, int(n))]
    return Workload("heavy_tail", seed, "bf16", num_blocks, block_size, num_heads,
                    num_kv_heads, head_dim, order, ops, decode_seqs=list(range(batch)),
                    outliers=True)


WORKLOADS = {
    "tiny_fp32": tiny_fp32,
    "gqa_decode": gqa_decode,
    "long_decode": long_decode,
    "prefix_prefill": prefix_prefill,
    "heavy_tail": heavy_tail,
}


# --------------------------------------------------------------- data streams
def append_stream(wl, only=None):
    """Yield each op of ``wl``; appends carry their K/V rows.

    Yields ``("create", s)``, ``("share", src, dst, prefix)`` and
    ``("append", s, n, k, v)`` where ``k, v`` have shape ``[n, Hkv, D]`` in the
    input dtype (bf16 bit patterns or float32).  With ``only`` (a set of
    sequence ids) the rows of other sequences are not drawn and are yielded
    as ``None``.
    """
    kv_rngs = {}
    out_rngs = {}
    shape_tail = (wl.num_kv_heads, wl.head_dim)
    for op in wl.ops:
        if op[0] != "append":
            yield op
            continue
        _, s, n = op
        if only is not None and s not in only:
            yield ("append", s, n, None, None)
            continue
        g = kv_rngs.setdefault(s, np.random.default_rng([wl.seed, 1, s]))
        k = g.standard_normal((n,) + shape_tail, dtype=np.float32)
        v = g.standard_normal((n,) + shape_tail, dtype=np.float32)
        if wl.outliers:
            go = out_rngs.setdefault(s, np.random.default_rng([wl.seed, 3, s]))
            mask = go.random((n, wl.num_kv_heads)) < 0.01
            k[mask] *= 8.0
            v[mask] *= 8.0
        yield ("append", s, n, _round(k, wl.dtype), _round(v, wl.dtype))



def decode_queries(wl, seqs=None):
    """Decode queries ``[B, Hq, D]`` (one row per listed decode sequence)."""
    seqs = wl.decode_seqs if seqs is None else seqs
    rows = []
    for s in seqs:
        g = np.random.default_rng([wl.seed, 2, s])
        rows.append(g.standard_normal((1, wl.num_heads, wl.head_dim), dtype=np.float32))
    q = np.concatenate(rows, axis=0) if rows else np.zeros((0, wl.num_heads, wl.head_dim), np.float32)
    return _round(q, wl.dtype)


def prefill_queries(wl):
    """Prefill queries ``[sum q_len, Hq, D]`` in the listed order.

    A sequence that also has a decode call draws its decode row first from
    the same generator.
    """
    chunks = []
    for s, q_len in wl.prefill:
        g = np.random.default_rng([wl.seed, 2, s])
        if s in wl.decode_seqs:
            g.standard_normal((1, wl.num_heads, wl.head_dim), dtype=np.float32)
        chunks.append(g.standard_normal((q_len, wl.num_heads, wl.head_dim), dtype=np.float32))
    q = np.concatenate(chunks, axis=0)
    return _round(q, wl.dtype)


def logical_kv(wl, seqs):
    """K/V rows of each sequence in ``seqs`` in logical (token) order.

    Returns ``{seq: (K, V)}`` with arrays ``[len, Hkv, D]`` in the input dtype.
    Built by replaying the op list: an append concatenates its rows, a share
    starts the target with the source's first ``prefix`` rows.
    """
    want = set(seqs)
    # Sources whose prefixes reach a wanted sequence must be drawn too.
    for op in reversed(wl.ops):
        if op[0] == "share" and op[2] in want:
            want.add(op[1])
    rows = {}
    for op in append_stream(wl, only=want):
        if op[0] == "create":
            if op[1] in want:
                rows[op[1]] = ([], [], 0)
        elif op[0] == "share":
            _, src, dst, prefix = op
            if dst in want:
                ks, vs, _ = rows[src]
                k = np.concatenate(ks, axis=0)[:prefix] if ks else None
                v = np.concatenate(vs, axis=0)[:prefix] if vs else None
                rows[dst] = ([k] if k is not None else [], [v] if v is not None else [], prefix)
        else:
            _, s, n, k, v = op
            if s in want:
                ks, vs, length = rows[s]
                rows[s] = (ks + [k], vs + [v], length + n)
    out = {}
    for s in seqs:
        ks, vs, _ = rows[s]
        out[s] = (np.concatenate(ks, axis=0), np.concatenate(vs, axis=0))
    return out


def prefix_trace_requests(users=100, turns=5):
    """Token-id requests of the prefix-caching trace on the vladkulikov.com
    notebook "Модуль 10" (prefix-caching cell): user u, turn t sends
    [100 + u % 10] + 0..30 + [1000 + u, 2000 + t] + 0..13 (48 ids), users
    outer, turns inner.  Returns ``[(user, turn, tokens)]``."""
    out = []
    for user in range(users):
        for turn in range(turns):
            tokens = [100 + user % 10] + list(range(31)) + [1000 + user, 2000 + turn] + list(range(14))
            out.append((user, turn, tokens))
    return out
