"""Paged-attention benchmark on one MI355X.

One step is one decode step of one attention layer over the whole batch,
one call of pa_decode_step: append one token to every sequence (host
bookkeeping and slot mapping), store the new K/V rows in their slots and
upload the plan (one kernel), then decode attention (split-K partial kernel,
log-sum-exp merge).  Workload: 32 sequences with lengths uniform in [1, 8192], 32 query /
8 KV heads, head_dim 128, bf16 K/V, block_size 16, a 32768-block pool with
shuffled block tables, Q/K/V ~ N(0, 1) (seeded, synthetic).  Successive steps
take the pools of ``--layers`` layers (default 8) in turn, as a model's layers
do, so a step never finds its pages in the 256 MB last-level cache from the
step before.

Printed: one JSON line.  ``value`` = decode KV GB/s over whole steps
(algorithmic bytes: every cached K and V row once, plus Q, O and the block
tables; decimal GB).  ``roofline`` covers the decode partial kernel alone,
timed with HIP events recorded on the stream it is launched on.
``int8_decode`` / ``fp8_decode`` repeat the decode steps over 8-bit pages
(int8 or E4M3 codes plus one fp32 scale per row).  ``prefill`` measures the chunked causal prefill of 16 sequences x 512 rows on
a shared 4096-token prefix (TFLOP/s on causal FLOPs).  ``cpu_baseline`` times
the float64 oracle on a bounded sample of the same decode workload.
"""

from __future__ import annotations

import argparse
import gc
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, decimal GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def to_device(arr, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def build_pool(wl, kv=None):
    """Replay ``wl`` into a DevicePool whose pages hold ``kv`` ("bf16", "f32",
    "i8" or "fp8"; default the workload's dtype).  New rows are in the
    workload's dtype either way (an 8-bit pool quantises them as it stores
    them)."""
    from paged_kv_cache_block_amd import DevicePool
    from synth import append_stream
    pool = DevicePool(wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim, dtype=kv or wl.dtype,
                      allocation_order=wl.allocation_order)
    for op in append_stream(wl):
        if op[0] == "create":
            pool.create(op[1])
        elif op[0] == "share":
            pool.share(*op[1:])
        else:
            _, s, n, k, v = op
            pool.write(pool.append(s, n), to_device(k, wl.dtype), to_device(v, wl.dtype))
    return pool


def build_layers(wl, kv, n_layers):
    """``n_layers`` pools of ``wl`` (one per model layer): the first replays
    the workload with its rows, the others replay the same bookkeeping (so
    the same block tables) and copy the first's pages."""
    from paged_kv_cache_block_amd import DevicePool
    import torch
    first = build_pool(wl, kv)
    pools = [first]
    for _ in range(n_layers - 1):
        p = DevicePool(wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim, dtype=kv or wl.dtype,
                       allocation_order=wl.allocation_order)
        for op in wl.ops:
            if op[0] == "create":
                p.create(op[1])
            elif op[0] == "share":
                p.share(*op[1:])
            else:
                p.append(op[1], op[2])
        p.flush()
        p.k.copy_(first.k)
        p.v.copy_(first.v)
        pools.append(p)
    torch.cuda.synchronize()
    return pools


def decode_alg_bytes(lengths, wl, kv_dtype=None):
    """K and V rows once each, plus Q, O and the block tables.  An 8-bit row
    is head_dim code bytes plus its 4-byte fp32 scale."""
    elt = wl.elt_bytes
    row = wl.head_dim + 4 if kv_dtype in ("i8", "fp8") else wl.head_dim * elt
    kv = sum(lengths) * wl.num_kv_heads * row * 2
    qo = 2 * len(lengths) * wl.num_heads * wl.head_dim * elt
    tables = sum(-(-n // wl.block_size) for n in lengths) * 4
    return kv + qo + tables


def causal_flops(wl):
    """4 * Hq * D per visible query-key pair (QK and PV, 2 FLOP per MAC)."""
    lengths = wl.final_lengths()
    total = 0
    for s, q_len in wl.prefill:
        prefix = lengths[s] - q_len
        total += 4 * wl.num_heads * wl.head_dim * (q_len * prefix + q_len * (q_len + 1) // 2)
    return total


def recorded_traffic(name):
    """HBM bytes per launch from the committed counter summary of a kernel,
    or None when the kernel's source has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", name + ".counters.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if decode_source_digest() != rec.get("kernel_code_sha256"):
        return None
    return rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]


def decode_source_digest(texts=None):
    """sha256 of the decode kernel's code and of the plan builder that sizes
    its launch (decode.hip, device.hpp, plan.cpp) with line comments,
    trailing blanks and empty lines removed, so that an edit of comments
    alone keeps the recorded counters."""
    import hashlib
    import re
    if texts is None:
        csrc = os.path.join(ROOT, "paged_kv_cache_block_amd", "csrc")
        texts = [open(os.path.join(csrc, f), encoding="utf-8").read()
                 for f in ("decode.hip", "device.hpp", "plan.cpp")]
    lines = []
    for text in texts:
        for line in text.splitlines():
            code = re.sub(r"//.*$", "", line).rstrip()
            if code:
                lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def window_alg_bytes(lengths, wl, sinks, recent):
    """Bytes of the keys a windowed decode row sees: min(L, sinks + recent)
    K and V rows per sequence, plus Q, O and the visited table entries."""
    seen = [min(int(n), sinks + recent) for n in lengths]
    kv = sum(seen) * wl.num_kv_heads * wl.head_dim * 2 * wl.elt_bytes
    qo = 2 * len(lengths) * wl.num_heads * wl.head_dim * wl.elt_bytes
    return kv + qo + sum(-(-n // wl.block_size) for n in seen) * 4


def settle():
    """Before the warmup of a timed loop: collect garbage (earlier legs'
    pools and tensors), then keep the collector off until ``unsettle``, so no
    collection lands inside the timed steps (the warmup re-warms what the
    collection evicted)."""
    gc.collect()
    gc.disable()


def unsettle():
    gc.enable()


SAMPLE_EVERY = 5  # timed steps that carry kernel timing events: one in this many


def device_copy_gbs(mib=1024, reps=10):
    """A plain device-to-device copy of ``mib`` MiB (context for the
    kernel figures): bytes read + written / time, decimal GB/s."""
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    b.synchronize()
    ms = a.elapsed_time(b) / reps
    return round(2 * (mib << 20) / (ms * 1e-3) / 1e9, 1)


def percentiles_us(samples_ms):
    """p10 / p50 / p90 of per-launch durations given in ms, in us."""
    if not samples_ms:
        return {}
    p10, p50, p90 = np.percentile(np.asarray(samples_ms) * 1e3, [10, 50, 90])
    return {"p10": round(float(p10), 2), "p50": round(float(p50), 2), "p90": round(float(p90), 2)}


def step_spread(step, indices):
    """Spread of the step time: the steps ``indices`` run back to back with
    one event recorded on the stream before each and one after the last;
    the interval between consecutive events is one step on the GPU's clock
    (the events add a few microseconds each, so the mean here sits above
    the event-free timed loop's)."""
    import torch
    indices = list(indices)
    if not indices:
        return {}
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(indices) + 1)]
    torch.cuda.synchronize()
    settle()
    for e, i in zip(evs, indices):
        e.record()
        step(i)
    evs[-1].record()
    evs[-1].synchronize()
    unsettle()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in zip(evs[:-1], evs[1:])])
    p10, p50, p90 = np.percentile(us, [10, 50, 90])
    return {"what": f"{len(us)} more steps, an event before each (adds its own few us)",
            "mean": round(float(us.mean()), 2), "p10": round(float(p10), 2), "p50": round(float(p50), 2),
            "p90": round(float(p90), 2), "max": round(float(us.max()), 2)}


def run_decode(args, kv="bf16", window=None, cold_steps=0):
    """Decode steps of workload 2 over ``args.layers`` layers' pools taken in
    turn (a step is one layer's pa_decode_step), so no step finds the pages it
    reads in a cache from an earlier step, as in a model whose layers each
    read their own cache once per token."""
    import torch
    from paged_kv_cache_block_amd import abi
    from synth import decode_queries, gqa_decode

    wl = gqa_decode()
    n_layers = max(1, args.layers)
    log(f"building the decode workload (32 x U[1,8192], 32/8 heads, d 128, {kv} pages, bs 16, "
        f"{n_layers} layers" + (f", window {window}" if window else "") + ")")
    pools = build_layers(wl, kv, n_layers)
    if window:
        for pool in pools:
            for s in wl.decode_seqs:
                pool.set_window(s, *window)
    seqs = list(wl.decode_seqs)
    B = len(seqs)
    q = to_device(decode_queries(wl), wl.dtype)
    out = torch.empty_like(q)
    # Every layer's pool takes at least one untimed step before the timed
    # loop, whatever --warmup is.
    warm = max(args.warmup, n_layers)
    total_steps = warm + args.steps
    extra_steps = 10  # after the timed region: merge / prologue kernel timing
    spread_steps = args.steps  # then the per-step spread, one event between steps
    gen = torch.Generator(device="cuda").manual_seed(1234)
    n_new = total_steps + extra_steps + spread_steps + cold_steps
    new_k = torch.randn((n_new, B, wl.num_kv_heads, wl.head_dim), generator=gen, device="cuda").to(torch.bfloat16)
    new_v = torch.randn((n_new, B, wl.num_kv_heads, wl.head_dim), generator=gen, device="cuda").to(torch.bfloat16)
    # lengths[l]: the sequence lengths of layer l's pool (each grows by 1 per step of that layer)
    lengths = [np.array([pool.seq_len(s) for s in seqs], dtype=np.int64) for pool in pools]
    # Workspace for the longest batch this run reaches (lengths grow by 1 a step).
    ws_need = abi.pa_decode_step_workspace_bytes(pools[0].handle, seqs, wl.num_heads)
    ws = torch.empty(2 * ws_need + (1 << 20), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    alg = []
    seq_arr = np.asarray(seqs, dtype=np.int64)
    handles = [pool.handle for pool in pools]
    ws_n = ws.numel()

    def step(i):
        # append 1 token per sequence + store its K/V + decode, one C call, on layer i % n_layers;
        # returns the lengths the call decoded over (its bytes are counted after the timed loop)
        layer = i % n_layers
        abi.pa_decode_step(handles[layer], seq_arr, wl.num_heads, new_k[i], new_v[i], q, out, ws, ws_n,
                           stream.cuda_stream)
        lengths[layer] += 1
        return lengths[layer].copy()

    def step_bytes(lens):
        return window_alg_bytes(lens, wl, *window) if window else decode_alg_bytes(lens, wl, kv)

    settle()
    log(f"warmup {warm} steps")
    for i in range(warm):
        step(i)
    torch.cuda.synchronize()
    abi.pa_timing_reset()
    # The decode kernel's duration comes from HIP events that its dispatch
    # carries, on every SAMPLE_EVERY-th timed step: a timed launch still
    # spaces the stream's kernels by a few microseconds, so the other steps
    # run untimed.  The merge and prologue kernels are timed in extra steps.
    abi.pa_timing_select([abi.PA_KERNEL_DECODE])
    log(f"timing {args.steps} steps")
    alg_timed = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    host_ms = []  # host time of each timed call (the call returns before its kernels finish)
    for j, i in enumerate(range(warm, total_steps)):
        timed = j % SAMPLE_EVERY == 0
        if timed:
            abi.pa_timing_enable(True)
        h0 = time.perf_counter()
        alg.append(step(i))
        host_ms.append((time.perf_counter() - h0) * 1e3)
        if timed:
            abi.pa_timing_enable(False)
            alg_timed.append(alg[-1])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    unsettle()
    alg = [step_bytes(x) for x in alg]
    alg_timed = [step_bytes(x) for x in alg_timed]
    dec_ms, dec_n = abi.pa_timing_read(abi.PA_KERNEL_DECODE)
    dec_pct = percentiles_us(abi.pa_timing_samples(abi.PA_KERNEL_DECODE))
    abi.pa_timing_select([abi.PA_KERNEL_MERGE, abi.PA_KERNEL_CACHE])
    abi.pa_timing_enable(True)
    for i in range(total_steps, total_steps + extra_steps):
        step(i)
    torch.cuda.synchronize()
    abi.pa_timing_enable(False)
    abi.pa_timing_select(None)
    mrg_ms, mrg_n = abi.pa_timing_read(abi.PA_KERNEL_MERGE)
    cache_ms, cache_n = abi.pa_timing_read(abi.PA_KERNEL_CACHE)
    first_spread = total_steps + extra_steps
    spread = step_spread(step, range(first_spread, first_spread + spread_steps))
    cold = None
    if cold_steps:
        # Cold caches: before each step a read of 1 GiB (outside the events)
        # evicts the 256 MB last-level cache and the L2s.  A read, not a
        # write: a write would leave dirty lines whose write-back then
        # competes with the decode's reads.
        flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        sink = torch.empty(cold_steps, dtype=torch.float32, device="cuda")
        abi.pa_timing_reset()
        abi.pa_timing_select([abi.PA_KERNEL_DECODE])
        abi.pa_timing_enable(True)
        cold_alg = []
        for c, i in enumerate(range(first_spread + spread_steps, n_new)):
            torch.sum(flush, dim=0, out=sink[c])
            cold_alg.append(step_bytes(step(i)))
        torch.cuda.synchronize()
        abi.pa_timing_enable(False)
        abi.pa_timing_select(None)
        samples = abi.pa_timing_samples(abi.PA_KERNEL_DECODE)
        del flush, sink
        c_ms = float(np.mean(samples))
        c_gbs = float(np.mean(cold_alg)) / (c_ms * 1e-3) / 1e9
        cold = {"what": "decode kernel after a 1 GiB device read that evicts the last-level cache and L2 "
                        f"({len(samples)} steps)",
                "decode_kernel_us": round(c_ms * 1e3, 2), **percentiles_us(samples),
                "GBs": round(c_gbs, 1), "frac": round(c_gbs / HBM_PEAK_GBS, 4)}
    for pool in pools:
        pool.validate()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    alg_per_step = float(np.mean(alg))
    kernel_ms = dec_ms / max(dec_n, 1)
    merge_ms = mrg_ms / max(mrg_n, 1)
    result = {
        "ms_per_step": ms_per_step,
        "value": alg_per_step / (ms_per_step * 1e-3) / 1e9,
        "tokens_per_s": B / (ms_per_step * 1e-3),
        "alg_bytes_per_step": alg_per_step,
        "decode_kernel_us": kernel_ms * 1e3,
        "merge_kernel_us": merge_ms * 1e3,
        "cache_kernel_us": cache_ms / max(cache_n, 1) * 1e3,
        "kernel_launches": {"decode": dec_n, "merge": mrg_n, "cache": cache_n},
        "decode_kernel_us_pct": dec_pct,
        "sum_len": int(lengths[0].sum()),
        "layers": n_layers,
        "host_call_ms": {"p50": round(float(np.median(host_ms)), 4), "max": round(float(np.max(host_ms)), 3),
                         "max_at_step": int(np.argmax(host_ms))},
        "step_us_pct": spread,
        "warmup_steps_run": warm,
    }
    if cold:
        result["cold_cache"] = cold
    achieved = float(np.mean(alg_timed)) / (kernel_ms * 1e-3) / 1e9
    kernel = {"i8": "decode_mfma_i8", "fp8": "decode_mfma_fp8"}.get(kv, "decode_mfma_bf16")
    traffic = recorded_traffic(f"{kernel}__gqa_decode")
    result["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                          "traffic": None if traffic is None else round(traffic / 1e9, 4),
                          "traffic_unit": "GB per launch",
                          "kernel": f"decode_mfma<128,16,1,{ {'i8': 'int8', 'fp8': 'e4m3'}.get(kv, 'bf16')}>",
                          "decode_plus_merge_GBs": round(alg_per_step / ((kernel_ms + merge_ms) * 1e-3) / 1e9, 1)}
    for pool in pools:
        pool.close()
    return wl, result


def run_verify(args, q_len=4):
    """Multi-token steps: every sequence of the decode workload appends and
    verifies ``q_len`` tokens per step (pa_verify_step); the K/V pages are
    read once for all q_len rows."""
    import torch
    from paged_kv_cache_block_amd import abi
    from synth import gqa_decode

    wl = gqa_decode()
    n_layers = max(1, args.layers)
    log(f"building the verify workload ({q_len} rows per sequence and step, {n_layers} layers)")
    pools = build_layers(wl, "bf16", n_layers)
    seqs = list(wl.decode_seqs)
    B = len(seqs)
    q_lens = [q_len] * B
    R = B * q_len
    warm = max(args.warmup, n_layers)  # every layer's pool takes an untimed step first
    total_steps = warm + args.steps
    n_new = total_steps + args.steps  # then the per-step spread
    gen = torch.Generator(device="cuda").manual_seed(4321)
    new_k = torch.randn((n_new, R, wl.num_kv_heads, wl.head_dim), generator=gen, device="cuda").to(torch.bfloat16)
    new_v = torch.randn((n_new, R, wl.num_kv_heads, wl.head_dim), generator=gen, device="cuda").to(torch.bfloat16)
    q = torch.randn((R, wl.num_heads, wl.head_dim), generator=gen, device="cuda").to(torch.bfloat16)
    out = torch.empty_like(q)
    lengths = [np.array([pool.seq_len(s) for s in seqs], dtype=np.int64) for pool in pools]
    need = abi.pa_verify_step_workspace_bytes(pools[0].handle, seqs, q_lens, wl.num_heads)
    ws = torch.empty(2 * need + (1 << 20), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    seq_arr = np.asarray(seqs, dtype=np.int64)
    ql_arr = np.asarray(q_lens, dtype=np.int32)
    handles = [pool.handle for pool in pools]
    ws_n = ws.numel()

    def step(i):
        layer = i % n_layers
        abi.pa_verify_step(handles[layer], seq_arr, ql_arr, wl.num_heads, new_k[i], new_v[i], q, out, ws, ws_n,
                           stream)
        lengths[layer] += q_len
        return lengths[layer].copy()

    def step_bytes(lens):
        return decode_alg_bytes(lens, wl) + 2 * (R - B) * wl.num_heads * wl.head_dim * wl.elt_bytes

    settle()
    for i in range(warm):
        step(i)
    torch.cuda.synchronize()
    abi.pa_timing_reset()
    abi.pa_timing_select([abi.PA_KERNEL_DECODE])
    alg = []
    t0 = time.perf_counter()
    for j, i in enumerate(range(warm, total_steps)):
        timed = j % SAMPLE_EVERY == 0
        if timed:
            abi.pa_timing_enable(True)
        a = step(i)
        if timed:
            abi.pa_timing_enable(False)
            alg.append(a)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    unsettle()
    abi.pa_timing_select(None)
    dec_ms, dec_n = abi.pa_timing_read(abi.PA_KERNEL_DECODE)
    spread = step_spread(step, range(total_steps, n_new))
    for pool in pools:
        pool.validate()
        pool.close()
    ms = (t1 - t0) * 1e3 / args.steps
    kernel_ms = dec_ms / max(dec_n, 1)
    return {"workload": f"gqa_decode with {q_len} query rows per sequence and step (pa_verify_step: "
                        f"append {q_len} tokens + store their K/V + causal attention)",
            "ms_per_step": round(ms, 5), "step_us_pct": spread, "rows_per_s": round(R / (ms * 1e-3), 1),
            "decode_kernel_us": round(kernel_ms * 1e3, 2),
            "kernel_GBs": round(float(np.mean([step_bytes(x) for x in alg])) / (kernel_ms * 1e-3) / 1e9, 1)}


def run_decode_only(args, name):
    """Decode kernels alone (pa_decode: plan upload, partial kernel, merge)
    on the long-context workload 3 or the heavy-tailed workload 5, whose
    pools are full or nearly so (no appends).  Every call is timed with
    dispatch-carried events; the figures are kernel GB/s on the algorithmic
    bytes."""
    import torch
    from paged_kv_cache_block_amd import abi
    from synth import decode_queries, heavy_tail, long_decode

    wl = long_decode() if name == "long" else heavy_tail()
    log(f"building {wl.name} ({sum(wl.final_lengths().values())} tokens)")
    pool = build_pool(wl)
    seqs = list(wl.decode_seqs)
    q = to_device(decode_queries(wl), wl.dtype)
    out = torch.empty_like(q)
    need = abi.pa_decode_workspace_bytes(pool.handle, seqs, wl.num_heads)
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    lengths = np.array([pool.seq_len(s) for s in seqs], dtype=np.int64)
    alg = decode_alg_bytes(lengths, wl)
    settle()
    for _ in range(args.warmup):
        abi.pa_decode(pool.handle, seqs, wl.num_heads, q, out, ws, ws.numel(), stream)
    torch.cuda.synchronize()
    abi.pa_timing_reset()
    abi.pa_timing_select([abi.PA_KERNEL_DECODE, abi.PA_KERNEL_MERGE])
    abi.pa_timing_enable(True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        abi.pa_decode(pool.handle, seqs, wl.num_heads, q, out, ws, ws.numel(), stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    unsettle()
    abi.pa_timing_enable(False)
    abi.pa_timing_select(None)
    d_ms, d_n = abi.pa_timing_read(abi.PA_KERNEL_DECODE)
    m_ms, m_n = abi.pa_timing_read(abi.PA_KERNEL_MERGE)
    d_pct = percentiles_us(abi.pa_timing_samples(abi.PA_KERNEL_DECODE))
    pool.close()
    k_ms = d_ms / max(d_n, 1)
    mg_ms = m_ms / max(m_n, 1)
    gbs = alg / (k_ms * 1e-3) / 1e9
    return {"workload": f"{wl.name}: {len(seqs)} seqs, sum of lengths {int(lengths.sum())}, "
                        f"{wl.num_heads}/{wl.num_kv_heads} heads, d {wl.head_dim}, bs {wl.block_size}, bf16",
            "alg_bytes": int(alg), "decode_kernel_us": round(k_ms * 1e3, 2), "decode_kernel_us_pct": d_pct,
            "merge_kernel_us": round(mg_ms * 1e3, 2), "kernel_GBs": round(gbs, 1),
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "decode_plus_merge_GBs": round(alg / ((k_ms + mg_ms) * 1e-3) / 1e9, 1),
            "ms_per_call": round((t1 - t0) * 1e3 / args.steps, 4),
            "tokens_per_s_kernels": round(len(seqs) / ((k_ms + mg_ms) * 1e-3), 1)}


def run_prefill(args, kv=None):
    """Chunked prefill of workload 4 (pages in ``kv``, default bf16)."""
    import torch
    from paged_kv_cache_block_amd import abi
    from synth import prefill_queries, prefix_prefill

    wl = prefix_prefill()
    log(f"building the prefill workload (16 x 512 rows on a shared 4096 prefix, {kv or wl.dtype} pages)")
    pool = build_pool(wl, kv)
    seqs = [s for s, _ in wl.prefill]
    q_lens = [n for _, n in wl.prefill]
    q = to_device(prefill_queries(wl), wl.dtype)
    out = torch.empty_like(q)
    need = abi.pa_prefill_workspace_bytes(pool.handle, seqs, q_lens, wl.num_heads)
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    settle()
    for _ in range(max(1, args.prefill_warmup)):
        abi.pa_prefill_chunk(pool.handle, seqs, q_lens, wl.num_heads, q, out, ws, ws.numel(), stream)
    torch.cuda.synchronize()
    abi.pa_timing_reset()
    abi.pa_timing_enable(True)
    t0 = time.perf_counter()
    for _ in range(args.prefill_iters):
        abi.pa_prefill_chunk(pool.handle, seqs, q_lens, wl.num_heads, q, out, ws, ws.numel(), stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    unsettle()
    abi.pa_timing_enable(False)
    k_ms, k_n = abi.pa_timing_read(abi.PA_KERNEL_PREFILL)
    k_pct = percentiles_us(abi.pa_timing_samples(abi.PA_KERNEL_PREFILL))
    flops = causal_flops(wl)
    kernel_ms = k_ms / max(k_n, 1)
    call_ms = (t1 - t0) * 1e3 / args.prefill_iters
    tflops = flops / (kernel_ms * 1e-3) / 1e12
    pool.close()
    return {
        "workload": "prefix_prefill: 16 seqs share 4096 prefix + 512 own rows, 32/8 heads, d 128, "
                    + {"i8": "int8 K/V pages (bf16 q, out)", "fp8": "E4M3 K/V pages (bf16 q, out)"}.get(kv, "bf16")
                    + ", bs 16",
        "causal_flops": flops,
        "ms_per_call": call_ms,
        "kernel_ms": kernel_ms,
        "kernel_us_pct": k_pct,
        "tflops": round(tflops, 2),
        "tokens_per_s": round(sum(q_lens) / (call_ms * 1e-3), 1),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4)},
    }


def run_prefix_cache(reps=20):
    """Host cost of prefix-hash block reuse through the C ABI: the 500-request
    trace of the "Модуль 10" notebook (100 users x 5 turns, 48-token requests,
    block size 16), each request attach + append + register + release, with
    one shared scope; the cache is cleared between repetitions."""
    from paged_kv_cache_block_amd import DevicePool
    from synth import prefix_trace_requests
    reqs = [r[2] for r in prefix_trace_requests()]
    pool = DevicePool(1024, 16, 8, 128, metadata_only=True)
    hits = cached = 0
    settle()
    t0 = time.perf_counter()
    for rep in range(reps):
        hits = cached = 0
        for i, tokens in enumerate(reqs):
            hit = pool.prefix_attach(i, tokens, "shared-public-template", "model-r1")
            pool.append(i, len(tokens) - hit)
            pool.prefix_register(i, tokens, "shared-public-template", "model-r1")
            pool.release(i)
            hits += hit > 0
            cached += hit
        pool.prefix_clear()
    dt = time.perf_counter() - t0
    unsettle()
    pool.close()
    n = reps * len(reqs)
    return {"workload": "notebook prefix trace: 500 requests x 48 tokens, block 16, shared scope, "
                        "attach + append + register + release per request (Python ctypes calls)",
            "requests_per_s": round(n / dt, 1), "us_per_request": round(dt / n * 1e6, 2),
            "hit_request_fraction": hits / len(reqs),
            "reused_input_fraction": round(cached / (48 * len(reqs)), 6)}


def run_cpu_baseline(wl, seconds):
    """The float64 oracle (gather through its pool, then attention) on the
    first sequences of the same decode workload, repeated for ~``seconds``."""
    import oracle
    from synth import append_stream, decode_queries
    from synth.workloads import to_f64
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    sample = [0, 1, 2, 3]
    lengths = wl.final_lengths()
    blocks = sum(-(-lengths[s] // wl.block_size) for s in sample)
    pool = oracle.Pool(blocks, wl.block_size, wl.num_kv_heads, wl.head_dim)
    for op in append_stream(wl, only=set(sample)):
        if op[0] == "append" and op[1] in sample:
            pool.create(op[1])
            pool.write(pool.append(op[1], op[2]), to_f64(op[3], wl.dtype), to_f64(op[4], wl.dtype))
    q = to_f64(decode_queries(wl, sample), wl.dtype)
    settle()
    t0 = time.perf_counter()
    reps = 0
    while True:
        for i, s in enumerate(sample):
            oracle.paged_attention(pool, s, q[i:i + 1])
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    unsettle()
    sample_lengths = [lengths[s] for s in sample]
    alg = decode_alg_bytes(sample_lengths, wl) * reps
    return {"value": round(alg / dt / 1e9, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"float64 oracle paged decode of sequences {sample} of the same workload "
                      f"(lengths {sample_lengths}, all 32 heads), {reps} repetitions in {dt:.1f} s",
            "tokens_per_s": round(len(sample) * reps / dt, 2)}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layers", type=int, default=8,
                    help="decode / verify steps take this many layers' pools in turn (one layer per step)")
    ap.add_argument("--prefill-iters", type=int, default=20)
    ap.add_argument("--prefill-warmup", type=int, default=10,
                    help="untimed prefill calls before the timed ones (the clock settles over the "
                         "first ~10 calls after the memory-bound decode legs)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--legs", default="int8,fp8,verify,window,long,heavy,prefix",
                    help="comma list of the legs after the headline decode leg: int8, fp8 (decode and "
                         "prefill over int8 / E4M3 pages), verify, window, long, heavy (decode kernels on "
                         "workloads 3 and 5), prefix (the bf16 prefill and the CPU baseline have their "
                         "own switches)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a known-size reference "
                         "for hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the paged-attention path "
              "here is single-GPU.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    from paged_kv_cache_block_amd import abi
    abi.load()

    if args.calibration_copy_mib:
        n = args.calibration_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {n} bytes read, {n} bytes written")
        del src, dst

    wl, dec = run_decode(args, cold_steps=10)
    line = {
        "metric": "paged-attn decode KV GB/s (% of HBM peak) + tokens/s; prefill TFLOP/s",
        "value": round(dec["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gqa_decode: 32 seqs, lengths U[1,8192] (seed 1), 32 query / 8 KV heads, "
                               "head_dim 128, bf16 K/V, block_size 16, 32768-block pool per layer; "
                               "step = one layer's pa_decode_step (append 1 token/seq + store its K/V + "
                               f"decode), {args.layers} layers' pools taken in turn so no step re-reads "
                               "pages an earlier step left in a cache",
                   "global_batch": 32, "seq_len": "U[1,8192]", "parallelism": "single GPU"},
        "tokens_per_s": round(dec["tokens_per_s"], 1),
        "hbm_frac_step": round(dec["value"] / HBM_PEAK_GBS, 4),
        "step_us_pct": dec["step_us_pct"],
        "decode": {k: dec[k] for k in ("decode_kernel_us", "decode_kernel_us_pct", "merge_kernel_us",
                                        "cache_kernel_us", "alg_bytes_per_step", "kernel_launches", "sum_len",
                                        "host_call_ms", "warmup_steps_run", "cold_cache") if k in dec},
        "roofline": dec["roofline"],
        "device_copy_GBs": device_copy_gbs(),
    }
    legs = {x.strip() for x in args.legs.split(",") if x.strip()}
    for leg, kv, what in (("int8", "i8", "int8"), ("fp8", "fp8", "E4M3")):
        if leg not in legs:
            continue
        _, q8 = run_decode(args, kv=kv)
        line[f"{leg}_decode"] = {
            "workload": f"the same decode steps over {what} K/V pages (one fp32 scale per token and "
                        "KV head row; bf16 q, out and new rows)",
            "ms_per_step": round(q8["ms_per_step"], 5),
            "step_us_pct": q8["step_us_pct"],
            "tokens_per_s": round(q8["tokens_per_s"], 1),
            "kv_GBs_step": round(q8["value"], 2),
            "decode": {k: q8[k] for k in ("decode_kernel_us", "decode_kernel_us_pct", "merge_kernel_us",
                                           "cache_kernel_us", "alg_bytes_per_step", "kernel_launches",
                                           "sum_len", "host_call_ms")},
            "roofline": q8["roofline"],
        }
    if "verify" in legs:
        line["verify_q4"] = run_verify(args, 4)
    if "long" in legs:
        line["long_decode"] = run_decode_only(args, "long")
    if "heavy" in legs:
        line["heavy_tail_decode"] = run_decode_only(args, "heavy")
    if "window" in legs:
        _, wdec = run_decode(args, kv="bf16", window=(4, 1024))
        line["window_decode"] = {
            "workload": "the same decode steps with a window on every sequence: 4 sink tokens + the "
                        "1024 most recent (pages outside released by the appends)",
            "ms_per_step": round(wdec["ms_per_step"], 5),
            "step_us_pct": wdec["step_us_pct"],
            "tokens_per_s": round(wdec["tokens_per_s"], 1),
            "decode_kernel_us": round(wdec["decode_kernel_us"], 2),
            "kernel_GBs": wdec["roofline"]["achieved"],
            "kv_GBs_step": round(wdec["value"], 2),
            "cache_kernel_us": round(wdec["cache_kernel_us"], 2),
            "host_call_ms": wdec["host_call_ms"],
        }
    if not args.no_prefill:
        line["prefill"] = run_prefill(args)
        if "int8" in legs:
            line["int8_prefill"] = run_prefill(args, kv="i8")
        if "fp8" in legs:
            line["fp8_prefill"] = run_prefill(args, kv="fp8")
    if "prefix" in legs:
        line["prefix_cache"] = run_prefix_cache()
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        line["cpu_baseline"] = run_cpu_baseline(wl, args.cpu_seconds)
        line["cpu_baseline"]["gpu_step_over_cpu"] = round(line["value"] / line["cpu_baseline"]["value"], 1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
