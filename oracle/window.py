"""Sliding-window attention with attention sinks, as the oracle defines it.

Test infrastructure only (see the package docstring).

Sources: vladkulikov.com notebook "Модуль 10. KV-кэши и эффективный
инференс":

* the eviction cell's streaming rule: a sequence keeps its first ``sinks``
  tokens and its latest tokens up to a fixed budget, everything when it is
  no longer than the budget; the sinks may not exceed the budget;
* the explicit window caches (``NumpyKVCacheExplicit`` with ``window``): a
  query attends over the cache it sees, and a rollback (``truncate``) cannot
  bring back evicted tokens.

Readings taken here:

* query row t of a sequence whose K/V rows cover positions ``[0, L)`` and
  whose last ``q_len`` positions are being queried is itself position
  ``L - q_len + t``; it sees the positions ``window_keep(L - q_len + t + 1,
  sinks, recent)`` (its causal prefix, then the window rule with budget
  ``sinks + recent``);
* positions whose rows were evicted are gone: a row sees the kept positions
  that are still resident (the explicit caches attend over what they hold).
"""

from __future__ import annotations

import numpy as np

from .attention import attention


def window_keep(length, sinks, recent):
    """Positions of a ``length``-token prefix that a window of ``sinks``
    leading tokens and ``recent`` latest tokens keeps (the streaming rule
    with budget ``sinks + recent``): position p stays when it is a sink, p <
    sinks, or one of the latest, p >= length - recent.  A prefix no longer
    than the budget keeps every position, since then length - recent <=
    sinks."""
    for name, value in (("length", length), ("sinks", sinks), ("recent", recent)):
        if isinstance(value, bool) or not isinstance(value, (int, np.integer)) or value < 0:
            raise ValueError(f"{name} must be a non-negative integer")
    if sinks + recent < 1:
        raise ValueError("the window must keep at least one position")
    first_recent = int(length) - int(recent)
    return tuple(p for p in range(int(length)) if p < sinks or p >= first_recent)


def windowed_attention(q, keys, values, positions, length, sinks, recent):
    """Attention of the last ``q.shape[0]`` positions of a ``length``-token
    sequence under a (sinks, recent) window.

    ``keys`` / ``values`` ``[n, Hkv, D]`` are the resident rows, at
    ``positions`` (ascending).  Row t uses the resident positions among
    ``window_keep(length - q_len + t + 1, sinks, recent)``.
    """
    q = np.asarray(q, dtype=np.float64)
    positions = list(positions)
    index = {p: i for i, p in enumerate(positions)}
    q_len = q.shape[0]
    out = np.empty_like(q)
    for t in range(q_len):
        kept = window_keep(length - q_len + t + 1, sinks, recent)
        rows = [index[p] for p in kept if p in index]
        if not rows:
            raise ValueError(f"row {t} sees no resident key")
        out[t] = attention(q[t:t + 1], keys[rows], values[rows])[0]
    return out
