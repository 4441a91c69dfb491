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
