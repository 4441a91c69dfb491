"""Attention definition of the oracle, in float64.

Test infrastructure only (see the package docstring).

:func:`attention` is the plain definition that paged attention must reach
(up to rounding order), as ferrum-kv 0.4.0 ``src/attention.rs``
``paged_attention`` states it: query rows ``t = 0 .. q_len-1`` are the last
``q_len`` positions of a sequence whose cached length is ``kv_len``; query
head ``h`` reads KV head ``h // (num_heads / num_kv_heads)``; scores are
``q . k / sqrt(head_dim)``; key ``j`` is masked (weight zero) when
``j > kv_len - q_len + t`` (bottom-right causal alignment, the same rule as
the ``CachedDecoder`` mask of CMU 11-667 lecture 19); weights are the
max-shifted softmax over the visible keys; the output is the weighted sum of
value rows, laid out ``[q_len, num_heads, head_dim]``.  A decode query is
``q_len = 1``: it sees every cached key (abhik.ai "examples/pagedattention.py",
region paged_attention).

The remaining functions restate the same quantity other ways, for
self-checks and for the split-K algebra:

* :func:`online_softmax_stats` / :func:`tiled_attention` -- the one-pass
  running-max recurrence of CMU 11-667 lecture 19 section 3 (per key block:
  ``m' = max(m, max s)``, rescale by ``exp(m - m')``, a block starting from
  ``m = -inf`` gets weight zero for its empty history);
* :func:`partial_attention` / :func:`merge_partials` -- unnormalised
  ``(m, l, acc)`` over a key range, and their log-sum-exp combination, which
  is the same recurrence applied across key ranges instead of key blocks;
* :func:`brute_force_attention` -- scalar Python loops in the order of
  ferrum-kv's ``paged_attention`` (tiny inputs only).

Readings where the pages are silent or differ: an empty cache
(``kv_len = 0``) is an error as in ferrum-kv (the first page returns zeros);
``q_len > kv_len`` and ``num_heads % num_kv_heads != 0`` are errors.
"""

from __future__ import annotations

import functools
import math

import numpy as np


def _check(q, K, V):
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if q.ndim != 3 or K.ndim != 3 or V.shape != K.shape:
        raise ValueError("q must be [q_len, Hq, D]; K, V must be [kv_len, Hkv, D]")
    q_len, num_heads, head_dim = q.shape
    kv_len, num_kv_heads, kdim = K.shape
    if kdim != head_dim:
        raise ValueError("head_dim mismatch")
    if kv_len == 0:
        raise ValueError("kv_len must be positive")
    if q_len == 0 or q_len > kv_len:
        raise ValueError("q_len must be in 1..kv_len")
    if num_heads % num_kv_heads:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    return q, K, V


def visible(kv_len, q_len, t):
    """Number of keys query row ``t`` may attend to (bottom-right causal)."""
    return kv_len - q_len + t + 1


def attention(q, K, V):
    """Softmax attention of ``q [q_len, Hq, D]`` over ``K, V [kv_len, Hkv, D]``."""
    q, K, V = _check(q, K, V)
    q_len, num_heads, head_dim = q.shape
    kv_len, num_kv_heads, _ = K.shape
    group = num_heads // num_kv_heads
    scale = 1.0 / math.sqrt(head_dim)
    key_pos = np.arange(kv_len)[None, :]
    row_pos = np.arange(q_len)[:, None]
    masked = key_pos > kv_len - q_len + row_pos          # [q_len, kv_len]
    out = np.empty((q_len, num_heads, head_dim))
    for h in range(num_heads):
        g = h // group
        s = (q[:, h, :] @ K[:, g, :].T) * scale          # [q_len, kv_len]
        s = np.where(masked, -np.inf, s)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h, :] = (p @ V[:, g, :]) / p.sum(axis=1, keepdims=True)
    return out


def paged_attention(pool, seq, q):
    """Attention of ``q`` (the last ``q_len`` positions of ``seq``) over the
    live K/V rows that the pool's block table gathers, in logical order."""
    K, V = pool.gather(seq)
    return attention(q, K, V)


def _score_stats(block):
    """(max, sum of exp(s - max)) of one block of scores; (-inf, 0) when
    the block is empty or wholly masked."""
    x = np.asarray(block, dtype=np.float64).ravel()
    top = float(x.max()) if x.size else -math.inf
    if top == -math.inf:
        return -math.inf, 0.0
    return top, float(np.exp(x - top).sum())


def combine_stats(a, b):
    """Statistics of the union of two score sets from theirs: the larger
    maximum, and each normaliser moved onto it by exp(m - max)."""
    top = max(a[0], b[0])
    if top == -math.inf:
        return -math.inf, 0.0
    return top, sum(l * math.exp(m - top) for m, l in (a, b) if m != -math.inf)


def online_softmax_stats(score_blocks):
    """Running (max, normaliser) over a stream of score blocks, folded one
    block at a time with :func:`combine_stats`; softmax(x)_i is then
    exp(x_i - max) / normaliser."""
    return functools.reduce(combine_stats, map(_score_stats, score_blocks), (-math.inf, 0.0))


def tiled_attention(q, K, V, block):
    """Same result as :func:`attention`, one key block at a time."""
    q, K, V = _check(q, K, V)
    q_len, num_heads, head_dim = q.shape
    kv_len, num_kv_heads, _ = K.shape
    group = num_heads // num_kv_heads
    scale = 1.0 / math.sqrt(head_dim)
    out = np.empty((q_len, num_heads, head_dim))
    row_pos = np.arange(q_len)[:, None]
    for h in range(num_heads):
        g = h // group
        m = np.full(q_len, -np.inf)
        l = np.zeros(q_len)
        acc = np.zeros((q_len, head_dim))
        for s0 in range(0, kv_len, block):
            keys = np.arange(s0, min(s0 + block, kv_len))[None, :]
            s = (q[:, h, :] @ K[keys[0], g, :].T) * scale
            s = np.where(keys > kv_len - q_len + row_pos, -np.inf, s)
            m_new = np.maximum(m, s.max(axis=1))
            # A row whose history and block are both fully masked keeps m = -inf;
            # its rescale factor is 0 and its block weights are 0.
            finite = np.isfinite(m_new)
            alpha = np.where(finite & np.isfinite(m), np.exp(np.where(finite, m - m_new, 0.0)), 0.0)
            p = np.where(finite[:, None], np.exp(s - np.where(finite, m_new, 0.0)[:, None]), 0.0)
            acc = acc * alpha[:, None] + p @ V[keys[0], g, :]
            l = l * alpha + p.sum(axis=1)
            m = m_new
        out[:, h, :] = acc / l[:, None]
    return out


def partial_attention(q, K, V, start, stop):
    """Unnormalised ``(m, l, acc)`` of each (row, head) over keys [start, stop).

    ``m [q_len, Hq]`` is the largest visible score in the range (``-inf`` if
    none is visible), ``l`` the sum of ``exp(s - m)`` and ``acc [q_len, Hq, D]``
    the matching weighted sum of value rows.
    """
    q, K, V = _check(q, K, V)
    q_len, num_heads, head_dim = q.shape
    kv_len, num_kv_heads, _ = K.shape
    group = num_heads // num_kv_heads
    scale = 1.0 / math.sqrt(head_dim)
    keys = np.arange(start, stop)
    masked = keys[None, :] > kv_len - q_len + np.arange(q_len)[:, None]
    m = np.full((q_len, num_heads), -np.inf)
    l = np.zeros((q_len, num_heads))
    acc = np.zeros((q_len, num_heads, head_dim))
    for h in range(num_heads):
        g = h // group
        s = (q[:, h, :] @ K[keys, g, :].T) * scale
        s = np.where(masked, -np.inf, s)
        for t in range(q_len):
            if keys.size == 0 or not np.isfinite(s[t]).any():
                continue
            m[t, h] = s[t].max()
            p = np.exp(s[t] - m[t, h])
            l[t, h] = p.sum()
            acc[t, h] = p @ V[keys, g, :]
    return m, l, acc


def merge_partials(ms, ls, accs):
    """Combine partial results of disjoint key ranges into the output.

    ``M = max_c m_c``; ``o = sum_c exp(m_c - M) acc_c / sum_c exp(m_c - M) l_c``;
    a range with ``m_c = -inf`` (nothing visible) weighs zero.
    """
    ms = np.asarray(ms, dtype=np.float64)
    ls = np.asarray(ls, dtype=np.float64)
    accs = np.asarray(accs, dtype=np.float64)
    big = ms.max(axis=0)
    w = np.where(np.isfinite(ms), np.exp(ms - big[None]), 0.0)
    num = (w[..., None] * accs).sum(axis=0)
    den = (w * ls).sum(axis=0)
    return num / den[..., None]


def brute_force_attention(q, K, V):
    """Scalar loops in ferrum-kv's order (query row, head, key): tiny inputs."""
    q, K, V = _check(q, K, V)
    q_len, num_heads, head_dim = q.shape
    kv_len, num_kv_heads, _ = K.shape
    group = num_heads // num_kv_heads
    scale = 1.0 / math.sqrt(head_dim)
    out = np.zeros((q_len, num_heads, head_dim))
    for t in range(q_len):
        for h in range(num_heads):
            g = h // group
            last = kv_len - q_len + t
            scores = []
            for j in range(kv_len):
                if j > last:
                    scores.append(-math.inf)
                    continue
                dot = 0.0
                for d in range(head_dim):
                    dot += float(q[t, h, d]) * float(K[j, g, d])
                scores.append(dot * scale)
            top = max(scores)
            weights = [math.exp(s - top) if s != -math.inf else 0.0 for s in scores]
            total = sum(weights)
            for j in range(kv_len):
                w = weights[j] / total
                for d in range(head_dim):
                    out[t, h, d] += w * float(V[j, g, d])
    return out
