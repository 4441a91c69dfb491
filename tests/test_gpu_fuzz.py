"""Seeded random-shape differential test of the attention calls on the GPU.

Each seed draws a geometry (page dtype bf16 / int8 / E4M3 / fp32, head_dim
64 or 128, block size 16 or 32, 1-8 KV heads, group 1-8), a batch of 1-5
sequences with log-uniform lengths, and a sliding window (sinks + recent)
on some of them; then, against the float64 oracle on the same rows:
decode of every sequence, a verify step with random row counts (the
MFMA page dtypes), and a prefill chunk of random length appended to every
sequence.  A child sharing a random prefix of one sequence (then growing
past it) and a fork of that sequence join the batch first, and two fused
decode steps run before the verify step, so copy-on-write of shared
partial tails happens inside the device calls.  The fixed cases of the
other GPU tests pin known shapes; this one walks shapes nobody picked by
hand.

Sources: docs.rs ferrum-kv 0.4.0 src/attention.rs, paged_attention (GQA,
scale, bottom-right causal mask for multi-token queries); vladkulikov.com
notebook "Модуль 10", eviction cell (the window keep rule) and the
KV-compression experiment (8-bit codes with fp32 row scales).  Bar: slots,
tables and refcounts bit-exact; outputs within (2e-3, 1e-2) of the oracle
((1e-5, 1e-5) for fp32 pools).
"""

import numpy as np
import pytest

import oracle
from synth.workloads import bf16_round, to_f64

from gpu_support import BF16_TOL, F32_TOL, assert_close, log, to_device, to_host_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SEEDS = list(range(32))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_block_amd import abi
    abi.load()


def _config(seed):
    rng = np.random.default_rng(1000 + seed)
    kv = ["bf16", "i8", "fp8", "f32"][seed % 4]
    d = int(rng.choice([64, 128]))
    bs = int(rng.choice([16, 32]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 4, 8]))
    batch = int(rng.integers(1, 6))
    lengths = [int(np.exp(rng.uniform(0.0, np.log(6000.0)))) for _ in range(batch)]
    windows = []
    for n in lengths:  # recent up to half the length, so most windows release pages
        if rng.random() < 0.5:
            windows.append((int(rng.choice([0, 4, 16])), int(rng.integers(16, max(17, n // 2 + 1)))))
        else:
            windows.append(None)
    return rng, kv, d, bs, hkv, hkv * group, lengths, windows


def _draw(rng, shape, io):
    x = rng.standard_normal(shape).astype(np.float32)
    return bf16_round(x) if io == "bf16" else x


def _append_rows(pool, ref, rng, s, n, hkv, d, io):
    """Append n rows to sequence s on both sides and store their K/V."""
    k, v = _draw(rng, (n, hkv, d), io), _draw(rng, (n, hkv, d), io)
    slots = pool.append(s, n)
    assert slots.tolist() == ref.append(s, n)
    pool.write(slots, to_device(k, io), to_device(v, io))
    ref.write(slots, to_f64(k, io), to_f64(v, io))


def _want(ref, s, q_rows, io):
    """The oracle's attention of q_rows as the last rows of sequence s over
    its resident keys (its window, when it has one)."""
    pos, keys, values = ref.resident(s)
    win = ref.windows.get(s)
    if win is None:
        return oracle.attention(to_f64(q_rows, io), keys, values)
    return oracle.windowed_attention(to_f64(q_rows, io), keys, values, pos, ref.lengths[s], *win)


@pytest.mark.parametrize("seed", SEEDS)
def test_random_shapes_match_oracle(seed):
    from paged_kv_cache_block_amd import DevicePool
    rng, kv, d, bs, hkv, hq, lengths, windows = _config(seed)
    io = "f32" if kv == "f32" else "bf16"
    tol = F32_TOL if kv == "f32" else BF16_TOL
    group = hq // hkv
    log(f"fuzz seed {seed}: {kv} d {d} bs {bs} heads {hq}/{hkv} lengths {lengths} windows {windows}")
    grow = 300 + 32  # prefill chunk and verify rows appended later, per sequence
    nb = int(sum(-(-(n + grow) // bs) + 2 for n in lengths) + 2 * (-(-(64 + grow) // bs) + 2) + 16)
    order = rng.permutation(nb).astype(np.int32)
    pool = DevicePool(nb, bs, hkv, d, dtype=kv, allocation_order=order)
    ref = oracle.Pool(nb, bs, hkv, d, allocation_order=order, quant_bits=8 if kv in ("i8", "fp8") else None,
                     quant_fp8=kv == "fp8")
    seqs = list(range(len(lengths)))
    for s, (n, win) in zip(seqs, zip(lengths, windows)):
        pool.create(s)
        ref.create(s)
        if win is not None:
            pool.set_window(s, *win)
            ref.set_window(s, *win)
        done = 0
        while done < n:  # appended in chunks, so windows release pages as they slide
            m = min(int(rng.integers(1, 400)), n - done)
            _append_rows(pool, ref, rng, s, m, hkv, d, io)
            done += m

    # A child sharing a random prefix of the first sequence without a window,
    # grown past it, and a fork of the same sequence.
    plain = [s for s, w in zip(seqs, windows) if w is None]
    if plain:
        src, child, fork = plain[0], len(lengths), len(lengths) + 1
        prefix = int(rng.integers(1, ref.lengths[src] + 1))
        pool.share(src, child, prefix)
        ref.share(src, child, prefix)
        _append_rows(pool, ref, rng, child, int(rng.integers(1, 64)), hkv, d, io)
        pool.fork(src, fork)
        ref.fork(src, fork)
        seqs += [child, fork]

    # Decode: one query row per sequence over its whole (or windowed) cache.
    q = _draw(rng, (len(seqs), hq, d), io)
    got = to_host_f64(pool.decode(seqs, to_device(q, io)))
    want = np.concatenate([_want(ref, s, q[b:b + 1], io) for b, s in enumerate(seqs)])
    assert_close(got, want, *tol, what=f"seed {seed} decode")

    # Two fused decode steps: append one token to every sequence, store its
    # K/V row and decode, in one call.
    for step in range(2):
        k, v = _draw(rng, (len(seqs), hkv, d), io), _draw(rng, (len(seqs), hkv, d), io)
        q = _draw(rng, (len(seqs), hq, d), io)
        out, slots = pool.decode_step(seqs, to_device(k, io), to_device(v, io), to_device(q, io))
        want_slots = []
        for s in seqs:
            want_slots += ref.append(s, 1)
        assert slots.tolist() == want_slots
        ref.write(want_slots, to_f64(k, io), to_f64(v, io))
        want = np.concatenate([_want(ref, s, q[b:b + 1], io) for b, s in enumerate(seqs)])
        assert_close(to_host_f64(out), want, *tol, what=f"seed {seed} decode step {step}")

    # Verify step: append + store + causal attention of 1..32/G rows.
    if kv != "f32":
        q_lens = [int(rng.integers(1, 32 // group + 1)) for _ in seqs]
        rows = sum(q_lens)
        k, v = _draw(rng, (rows, hkv, d), io), _draw(rng, (rows, hkv, d), io)
        q = _draw(rng, (rows, hq, d), io)
        out, slots = pool.verify_step(seqs, q_lens, to_device(k, io), to_device(v, io), to_device(q, io))
        want_slots = []
        for s, n in zip(seqs, q_lens):
            want_slots += ref.append(s, n)
        assert slots.tolist() == want_slots
        ref.write(want_slots, to_f64(k, io), to_f64(v, io))
        got = to_host_f64(out)
        want, r0 = [], 0
        for s, n in zip(seqs, q_lens):
            want.append(_want(ref, s, q[r0:r0 + n], io))
            r0 += n
        assert_close(got, np.concatenate(want), *tol, what=f"seed {seed} verify {q_lens}")

    # Prefill: a chunk of 1..300 rows appended to every sequence, then its
    # causal attention (MFMA prefill, or the split-K kernels for short ones).
    q_lens = [int(rng.integers(1, 301)) for _ in seqs]
    for s, n in zip(seqs, q_lens):
        _append_rows(pool, ref, rng, s, n, hkv, d, io)
    q = _draw(rng, (sum(q_lens), hq, d), io)
    got = to_host_f64(pool.prefill(seqs, q_lens, to_device(q, io)))
    want, r0 = [], 0
    for s, n in zip(seqs, q_lens):
        want.append(_want(ref, s, q[r0:r0 + n], io))
        r0 += n
    assert_close(got, np.concatenate(want), *tol, what=f"seed {seed} prefill {q_lens}")

    for s in seqs:
        assert pool.block_table(s).tolist() == ref.tables[s]
    assert [pool.refcount(b) for b in range(ref.num_blocks)] == ref.refs.tolist()
    pool.validate()
    pool.close()
