"""Helpers for the GPU parity tests: replay a workload into a DevicePool and
compute the oracle's expected outputs from the same seeded inputs."""

from __future__ import annotations

import sys
import time

import numpy as np

import oracle
from synth import append_stream, logical_kv
from synth.workloads import to_f64


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


# ------------------------------------------------------------ page layouts
# The byte / element places of a page's values as the C header documents
# them, written out here from that text (the tests read device pages
# through these, independently of the library's own index code).
def k16_index(bs, d):
    """[bs, d] element offsets of a bf16 K page: with bs % 16 == 0 and
    d % 32 == 0, values d' = 32j + 8grp .. +7 of token t sit at
    (t // 16) * 16 d + (j * 64 + grp * 16 + t % 16) * 8 (+ d' % 8); other
    shapes are row-major."""
    t = np.arange(bs)[:, None]
    j = np.arange(d)[None, :]
    if bs % 16 or d % 32:
        return t * d + j
    return (t // 16) * 16 * d + ((j // 32) * 64 + (j % 32) // 8 * 16 + t % 16) * 8 + j % 8


def k8_index(bs, d):
    """[bs, d] byte offsets of the K codes of an 8-bit page: with d % 64 ==
    0, lane span s = d / 4, grp = d' // s, c = d' % s, chunk w = c // 16:
    (t // 16) * 16 d + (w * 64 + grp * 16 + t % 16) * 16 + c % 16;
    otherwise row-major."""
    t = np.arange(bs)[:, None]
    j = np.arange(d)[None, :]
    if d % 64:
        return t * d + j
    span = d // 4
    grp, c = j // span, j % span
    return (t // 16) * 16 * d + ((c // 16) * 64 + grp * 16 + t % 16) * 16 + c % 16


def v8_index(bs, d):
    """[bs, d] byte offsets of the V codes of an 8-bit page: row r = (t % 16)
    // 4 * 16 + d' % 16, byte c = (d' // 16) * 4 + t % 4 of the row; with
    d % 64 == 0 at (t // 16) * 16 d + ((c // 16) * 64 + r) * 16 + c % 16,
    otherwise at (t // 16) * 16 d + r * d / 4 + c."""
    t = np.arange(bs)[:, None]
    j = np.arange(d)[None, :]
    r = (t % 16) // 4 * 16 + j % 16
    c = (j // 16) * 4 + t % 4
    if d % 64:
        return (t // 16) * 16 * d + r * (d // 4) + c
    return (t // 16) * 16 * d + ((c // 16) * 64 + r) * 16 + c % 16


def to_device(arr, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def to_host_f64(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def build_device_pool(wl, check_against_oracle_pool=False):
    """Replay ``wl``'s ops into a DevicePool; optionally mirror them in the
    oracle pool (bookkeeping only) and compare slots after every append."""
    import torch
    from paged_kv_cache_block_amd import DevicePool
    pool = DevicePool(wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim, dtype=wl.dtype,
                      allocation_order=wl.allocation_order)
    ref = oracle.Pool(wl.num_blocks, wl.block_size, allocation_order=wl.allocation_order,
                      store_values=False) if check_against_oracle_pool else None
    for op in append_stream(wl):
        if op[0] == "create":
            pool.create(op[1])
            if ref:
                ref.create(op[1])
        elif op[0] == "share":
            pool.share(op[1], op[2], op[3])
            if ref:
                ref.share(op[1], op[2], op[3])
        else:
            _, s, n, k, v = op
            slots = pool.append(s, n)
            if ref:
                assert slots.tolist() == ref.append(s, n)
            pool.write(slots, to_device(k, wl.dtype), to_device(v, wl.dtype))
    torch.cuda.synchronize()
    return pool, ref


def build_device_pool_keeping_rows(wl):
    """``build_device_pool`` that also returns every sequence's K/V rows in
    logical order (``{seq: (K, V)}`` in the input dtype, as
    ``synth.logical_kv`` gives them), from the same single draw."""
    import torch
    from paged_kv_cache_block_amd import DevicePool
    pool = DevicePool(wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim, dtype=wl.dtype,
                      allocation_order=wl.allocation_order)
    parts = {}
    for op in append_stream(wl):
        if op[0] == "create":
            pool.create(op[1])
            parts[op[1]] = []
        elif op[0] == "share":
            _, src, dst, prefix = op
            pool.share(src, dst, prefix)
            taken, need = [], prefix
            for k, v in parts[src]:
                if need <= 0:
                    break
                taken.append((k[:need], v[:need]))
                need -= len(k)
            parts[dst] = taken
        else:
            _, s, n, k, v = op
            pool.write(pool.append(s, n), to_device(k, wl.dtype), to_device(v, wl.dtype))
            parts[s].append((k, v))
    torch.cuda.synchronize()
    rows = {s: (np.concatenate([k for k, _ in p]), np.concatenate([v for _, v in p])) for s, p in parts.items() if p}
    return pool, rows


def expected_decode(wl, seqs, q_bits):
    """Oracle output for one query row per sequence (float64)."""
    rows = logical_kv(wl, sorted(set(seqs)))
    out = {}
    for i, s in enumerate(seqs):
        K, V = rows[s]
        q = to_f64(q_bits[i:i + 1], wl.dtype)
        out[i] = oracle.attention(q, to_f64(K, wl.dtype), to_f64(V, wl.dtype))[0]
    return out


def assert_close(got, want, atol, rtol, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    err = np.abs(got - want)
    bound = atol + rtol * np.abs(want)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    ok = bool((err <= bound).all()) and np.isfinite(got).all()
    assert ok, (f"{what}: max abs err {err.max():.3e}, worst at {worst}: got {got[worst]!r} "
                f"want {want[worst]!r} (atol {atol}, rtol {rtol})")
    return float(err.max())


# Tolerances (elementwise |gpu - oracle| <= atol + rtol |oracle|): bf16 K/V
# with fp32 accumulation and bf16 output; fp32 everywhere.
BF16_TOL = (2e-3, 1e-2)
F32_TOL = (1e-5, 1e-5)


def tol(wl):
    return BF16_TOL if wl.dtype == "bf16" else F32_TOL
