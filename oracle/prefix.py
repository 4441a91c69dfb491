"""Prefix-hash block reuse over the oracle pool.

Test infrastructure only (see the package docstring).

Source: vladkulikov.com notebook "Модуль 10. KV-кэши и эффективный
инференс", the prefix-caching cell (its block keys and ``run_prefix_trace``)
and the context / model-revision identity checks after it.

* A cache key exists only at a complete block boundary ``end`` (a multiple of
  the block size) and is the triple (scope, revision, every token id before
  ``end``): the same block content after a different context, or under
  another model revision or scope, is a different key.
* A request's hit is the longest run of consecutive complete-block keys, from
  the first block on, that the cache holds (the walk stops at the first
  miss); afterwards every complete-block key of the request is added.

Readings taken here (the notebook's cache is a set of keys with no pool):

* each key maps to the physical block holding the block that ends at
  ``end``; the cache keeps one reference (a pool pin) per key, so a cached
  block outlives the sequences that wrote it;
* ``attach`` gives a new sequence the cached blocks of its hit (refcount + 1
  each, as a shared prefix) with length = hit; the caller appends and stores
  the rest;
* ``register`` adds the keys of a sequence's complete blocks once their K/V
  are stored, up to the first page a sliding window released; a key already
  present keeps its block (adding to a set);
* the notebook has no eviction; ``clear`` drops every key and its pin.
"""

from __future__ import annotations

from typing import NamedTuple

from .pool import HOLE


class BlockKey(NamedTuple):
    """Identity of the complete block ending at token index ``end`` of a
    request: its scope and model revision, and the ids of every token before
    ``end`` (so the same block content after another context is another
    key)."""

    scope: str
    revision: str
    context: tuple


def block_key(scope, revision, tokens, end):
    """:class:`BlockKey` of the complete block ending at ``end`` (a multiple
    of the block size, at most ``len(tokens)``)."""
    if not 0 < end <= len(tokens):
        raise ValueError("a block key ends inside the request")
    return BlockKey(scope, revision, tuple(int(t) for t in tokens[:end]))


class PrefixCache:
    """Complete-block prefix keys -> physical blocks of an oracle Pool."""

    def __init__(self, pool):
        self.pool = pool
        self.entries = {}

    def lookup(self, tokens, scope, revision):
        """Tokens covered by the longest run of cached complete blocks."""
        bs = self.pool.block_size
        hit = 0
        for end in range(bs, len(tokens) + 1, bs):
            if block_key(scope, revision, tokens, end) not in self.entries:
                break
            hit = end
        return hit

    def attach(self, seq, tokens, scope, revision):
        """New sequence holding the cached blocks of its hit; returns the hit."""
        bs = self.pool.block_size
        hit = self.lookup(tokens, scope, revision)
        blocks = [self.entries[block_key(scope, revision, tokens, end)]
                  for end in range(bs, hit + 1, bs)]
        self.pool.adopt(seq, blocks, hit)
        return hit

    def register(self, seq, tokens, scope, revision):
        """Add the keys of ``seq``'s complete blocks (``tokens`` are its first
        ``len(tokens)`` token ids); returns the number of new keys."""
        pool = self.pool
        bs = pool.block_size
        if len(tokens) > pool.sequence_length(seq):
            raise ValueError("more tokens than the sequence holds")
        table = pool.tables[seq]
        added = 0
        for end in range(bs, len(tokens) + 1, bs):
            if table[end // bs - 1] == HOLE:
                break  # keys stop at the first page a window released
            key = block_key(scope, revision, tokens, end)
            if key in self.entries:
                continue
            block = table[end // bs - 1]
            pool.pin(block)
            self.entries[key] = block
            added += 1
        return added

    def clear(self):
        """Drop every key and its pin; returns how many keys there were."""
        n = len(self.entries)
        for block in self.entries.values():
            self.pool.unpin(block)
        self.entries.clear()
        return n


def run_prefix_trace(pool, requests, scope_of, revision="model-r1"):
    """Serve ``requests`` (token lists) in order through a fresh cache on
    ``pool``: attach, append the uncached rest, register, release.

    Returns ``(hit_request_fraction, reused_input_fraction, cache)``.
    """
    cache = PrefixCache(pool)
    hit_requests = cached = total = 0
    for i, tokens in enumerate(requests):
        scope = scope_of(i)
        hit = cache.attach(("req", i), tokens, scope, revision)
        pool.append(("req", i), len(tokens) - hit)
        cache.register(("req", i), tokens, scope, revision)
        pool.release(("req", i))
        hit_requests += hit > 0
        cached += hit
        total += len(tokens)
    return hit_requests / len(requests), cached / total, cache
