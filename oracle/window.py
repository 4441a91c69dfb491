"""Sliding-window attention with attention sinks, as the oracle defines it.

Test infrastructure only (see the package docstring).

Sources: vladkulikov.com notebook "Модуль 10. KV-кэши и эффективный
инференс":

* the eviction cell, ``streaming_keep_indices(length, budget, sink_tokens)``:
  with ``n = length`` tokens and ``budget`` kept, a sequence no longer than
  the budget keeps everything; otherwise the first ``min(sinks, n)`` tokens
  (the sinks) and the most recent ``budget - sinks`` tokens; ``sinks`` may
  not exceed the budget;
* the explicit window caches (``NumpyKVCacheExplicit`` with ``window``): a
  query attends over the cache it sees, and a rollback (``truncate``) cannot
  bring back evicted tokens.

Readings taken here:

* query row t of a sequence whose K/V rows cover positions ``[0, L)`` and
  whose last ``q_len`` positions are being queried is itself position
  ``L - q_len + t``; it sees the positions ``streaming_keep_indices(L -
  q_len + t + 1, sinks + recent, sinks)`` (its causal prefix, then the
  window rule);
* positions whose rows were evicted are gone: a row sees the kept positions
  that are still resident (the explicit caches attend over what they hold).
"""

from __future__ import annotations

import numpy as np

from .attention import attention


def streaming_keep_indices(length, budget, sink_tokens):
    """Kept positions of a ``length``-token sequence under ``budget``."""
    for name, value, low in (("length", length, 0), ("budget", budget, 1), ("sink_tokens", sink_tokens, 0)):
        if isinstance(value, bool) or not isinstance(value, (int, np.integer)) or value < low:
            raise ValueError(f"{name} must be an integer >= {low}")
    n, keep, sinks = int(length), int(budget), int(sink_tokens)
    if sinks > keep:
        raise ValueError("sink_tokens cannot exceed budget")
    if n <= keep:
        return tuple(range(n))
    sink_count = min(sinks, n)
    recent_count = keep - sink_count
    recent_start = max(sink_count, n - recent_count)
    return tuple(range(sink_count)) + tuple(range(recent_start, n))


def windowed_attention(q, keys, values, positions, length, sinks, recent):
    """Attention of the last ``q.shape[0]`` positions of a ``length``-token
    sequence under a (sinks, recent) window.

    ``keys`` / ``values`` ``[n, Hkv, D]`` are the resident rows, at
    ``positions`` (ascending).  Row t uses the resident positions among
    ``streaming_keep_indices(length - q_len + t + 1, sinks + recent, sinks)``.
    """
    q = np.asarray(q, dtype=np.float64)
    positions = list(positions)
    index = {p: i for i, p in enumerate(positions)}
    q_len = q.shape[0]
    out = np.empty_like(q)
    for t in range(q_len):
        kept = streaming_keep_indices(length - q_len + t + 1, sinks + recent, sinks)
        rows = [index[p] for p in kept if p in index]
        if not rows:
            raise ValueError(f"row {t} sees no resident key")
        out[t] = attention(q[t:t + 1], keys[rows], values[rows])[0]
    return out
