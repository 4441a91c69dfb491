"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Bar: block tables, slots and refcounts bit-exact; attention outputs within
|gpu - oracle| <= atol + rtol |oracle| elementwise, (2e-3, 1e-2) for bf16
K/V with fp32 accumulation and bf16 output, (1e-5, 1e-5) for fp32.
Small instances of every workload are compared element by element; the
full-size workloads are compared on every output they have (decode at
32 x 8192) or on sampled sequences / query rows the oracle computes one by
one (131072-token and heavy-tailed decode, 4096-prefix prefill).
"""

import numpy as np
import pytest

import oracle
from synth import (append_stream, decode_queries, gqa_decode, heavy_tail, logical_kv,
                   long_decode, prefill_queries, prefix_prefill, tiny_fp32)
from synth.workloads import Workload, bf16_round, to_f64

from gpu_support import (build_device_pool_keeping_rows, BF16_TOL, F32_TOL, assert_close, build_device_pool, expected_decode, log,
                         to_device, to_host_f64, tol, k16_index)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_block_amd import abi
    abi.load()   # fail loudly if the library is missing


def _gather_pool_rows(pool, seq, length):
    """Live K/V rows of ``seq`` read back from the device pools through the
    documented layout (K pages: fp32 row-major [bs][D], bf16 in the page
    order of ``k16_index``; V pages [D][bs])."""
    table = pool.block_table(seq)
    bs, d = pool.block_size, pool.head_dim
    k = pool.k.float().cpu().numpy().reshape(pool.num_blocks, pool.num_kv_heads, bs * d)
    v = pool.v.float().cpu().numpy()
    kidx = k16_index(bs, d) if pool.dtype == "bf16" else np.arange(bs * d).reshape(bs, d)
    K = np.stack([k[table[p // bs]][:, kidx[p % bs]] for p in range(length)])
    V = np.stack([v[table[p // bs], :, :, p % bs] for p in range(length)])
    return K, V


def _decode(pool, wl, seqs):
    q_bits = decode_queries(wl, seqs)
    q = to_device(q_bits, wl.dtype)
    out = pool.decode(seqs, q)
    torch.cuda.synchronize()
    return q_bits, to_host_f64(out)


# ------------------------------------------------------------ workload 1
def test_tiny_fp32_workload():
    wl = tiny_fp32()
    log("tiny_fp32: build")
    pool, ref = build_device_pool(wl, check_against_oracle_pool=True)
    assert pool.block_table(0).tolist() == [2, 4] and pool.block_table(1).tolist() == [2, 3, 6]
    assert [pool.refcount(b) for b in range(8)] == ref.refs.tolist()
    assert pool.stats() == ref.stats()
    # The copy-on-write copy ran on the device before B's rows were written.
    rows = logical_kv(wl, [0, 1])
    for s, n in ((0, 6), (1, 9)):
        K, V = _gather_pool_rows(pool, s, n)
        np.testing.assert_array_equal(K, rows[s][0])
        np.testing.assert_array_equal(V, rows[s][1])
    log("tiny_fp32: decode")
    q_bits, got = _decode(pool, wl, [0, 1])
    want = expected_decode(wl, [0, 1], q_bits)
    for i in range(2):
        assert_close(got[i], want[i], *F32_TOL, what=f"decode seq {i}")
    log("tiny_fp32: prefill")
    qp = prefill_queries(wl)
    out = to_host_f64(pool.prefill([1], [3], to_device(qp, wl.dtype)))
    K, V = (to_f64(x, wl.dtype) for x in rows[1])
    exp = oracle.attention(to_f64(qp, wl.dtype), K, V)
    assert_close(out, exp, *F32_TOL, what="prefill")
    np.testing.assert_allclose(exp, oracle.brute_force_attention(to_f64(qp, wl.dtype), K, V), atol=1e-13)


# ------------------------------------------------------------ closed forms
def _f32_pool(keys, values, block_size, num_blocks, order=None):
    from paged_kv_cache_block_amd import DevicePool
    keys = np.asarray(keys, np.float32)
    n, hkv, d = keys.shape
    pool = DevicePool(num_blocks, block_size, hkv, d, dtype="f32", allocation_order=order)
    pool.create(0)
    slots = pool.append(0, n)
    pool.write(slots, torch.tensor(keys).cuda(), torch.tensor(np.asarray(values, np.float32)).cuda())
    return pool


def test_ferrum_closed_forms_on_gpu():
    import math
    heads, dim = 2, 4
    pool = _f32_pool(np.ones((3, heads, dim)),
                     np.stack([np.full((heads, dim), p + 1.0) for p in range(3)]), 16, 4)
    out = pool.decode([0], torch.ones(1, heads, dim).cuda()).cpu().numpy()
    np.testing.assert_allclose(out, 2.0, atol=1e-5)
    rows = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])[:, None, :]
    pool = _f32_pool(rows, rows, 16, 2)
    out = pool.prefill([0], [3], torch.tensor(rows, dtype=torch.float32).cuda()).cpu().numpy()[:, 0]
    w1 = 1.0 / (1.0 + math.exp(-1.0 / math.sqrt(2.0)))
    e = math.exp(1.0 / math.sqrt(2.0))
    np.testing.assert_allclose(out, [[1, 0], [1 - w1, w1], [(1 + e) / (2 + e)] * 2], atol=1e-5)
    keys = np.stack([np.full((1, 2), p + 1.0) for p in range(4)])
    pool = _f32_pool(keys, 10 * keys, 2, 4, order=[3, 1, 0, 2])
    out = pool.decode([0], torch.ones(1, 1, 2).cuda()).cpu().numpy()[0, 0]
    w = np.exp(np.sqrt(2.0) * np.arange(1, 5))
    np.testing.assert_allclose(out, [10 * (np.arange(1, 5) * w).sum() / w.sum()] * 2, rtol=1e-5)


# ------------------------------------------------------------ decode shapes
def _decode_case(lengths, hq, hkv, d, bs, dtype="bf16", seed=5, num_blocks=None, outliers=False):
    nb = num_blocks or int(sum(-(-n // bs) for n in lengths) + 7)
    order = np.random.default_rng(seed).permutation(nb).astype(np.int32)
    ops = []
    for i, n in enumerate(lengths):
        ops += [("create", i), ("append", i, int(n))]
    return Workload("case", seed, dtype, nb, bs, hq, hkv, d, order, ops,
                    decode_seqs=list(range(len(lengths))), outliers=outliers)


DECODE_CASES = [
    # lengths, Hq, Hkv, D, bs
    ([1, 2, 15, 16, 17, 33, 200, 700], 32, 8, 128, 16),      # GQA 4, ragged tails
    ([1, 64, 129, 1000, 4100], 64, 8, 128, 16),              # GQA 8, split-K
    ([5, 31, 32, 33, 517, 2049], 16, 16, 64, 32),             # MHA, D 64, bs 32
    ([3, 100, 1500], 16, 1, 128, 16),                         # GQA 16
    ([7, 77, 777], 8, 4, 64, 16),                             # GQA 2, D 64
    ([9, 300, 3000], 16, 2, 128, 32),                         # GQA 8, bs 32
    ([2, 90, 1200], 6, 2, 32, 8),                             # generic kernel (D 32, bs 8)
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"L{max(c[0])}-G{c[1]//c[2]}-D{c[3]}-bs{c[4]}")
def test_decode_shapes(case):
    lengths, hq, hkv, d, bs = case
    wl = _decode_case(lengths, hq, hkv, d, bs)
    log(f"decode case {case}: build")
    pool, ref = build_device_pool(wl, check_against_oracle_pool=True)
    seqs = list(range(len(lengths)))
    q_bits, got = _decode(pool, wl, seqs)
    want = expected_decode(wl, seqs, q_bits)
    for i in seqs:
        assert_close(got[i], want[i], *BF16_TOL, what=f"seq {i} (L={lengths[i]})")


def test_decode_fp32_generic():
    wl = _decode_case([1, 5, 40, 333], 4, 2, 16, 4, dtype="f32")
    pool, _ = build_device_pool(wl)
    q_bits, got = _decode(pool, wl, [0, 1, 2, 3])
    want = expected_decode(wl, [0, 1, 2, 3], q_bits)
    for i in range(4):
        assert_close(got[i], want[i], *F32_TOL, what=f"seq {i}")


def test_decode_batch_with_duplicates_and_shared_prefix():
    wl = prefix_prefill(batch=3, prefix=50, chunk=9, num_blocks=64, num_heads=32, num_kv_heads=8,
                        head_dim=128, block_size=16)
    pool, ref = build_device_pool(wl, check_against_oracle_pool=True)
    seqs = [2, 0, 2, 1]
    q_bits, got = _decode(pool, wl, seqs)
    want = expected_decode(wl, seqs, q_bits)
    for i in range(4):
        assert_close(got[i], want[i], *BF16_TOL, what=f"row {i}")
    assert (got[0] == got[2]).all()


@pytest.mark.parametrize("shape", [(32, 8, 128, 16), (16, 16, 64, 32), (4, 2, 8, 4)],
                         ids=["G4-D128-bs16", "G1-D64-bs32", "generic-fp32"])
def test_decode_step_matches_oracle(shape):
    """Fused step = batched append + cache write + decode, five steps in a
    row; sequence 3 is a fork of 0, so the first step copies a shared tail."""
    from paged_kv_cache_block_amd import DevicePool
    hq, hkv, d, bs = shape
    dtype = "f32" if d == 8 else "bf16"
    tol_ = F32_TOL if dtype == "f32" else BF16_TOL
    nb = 128
    order = np.random.default_rng(21).permutation(nb).astype(np.int32)
    pool = DevicePool(nb, bs, hkv, d, dtype=dtype, allocation_order=order)
    ref = oracle.Pool(nb, bs, hkv, d, allocation_order=order)
    rng = np.random.default_rng(5)

    def draw(shape_):
        x = rng.standard_normal(shape_).astype(np.float32)
        return bf16_round(x) if dtype == "bf16" else x

    for s, n in enumerate([37, 15, 200]):
        pool.create(s)
        ref.create(s)
        k, v = draw((n, hkv, d)), draw((n, hkv, d))
        slots = pool.append(s, n)
        assert slots.tolist() == ref.append(s, n)
        pool.write(slots, to_device(k, dtype), to_device(v, dtype))
        ref.write(slots, to_f64(k, dtype), to_f64(v, dtype))
    pool.fork(0, 3)
    ref.fork(0, 3)
    seqs = [0, 1, 2, 3]
    for step in range(5):
        k, v = draw((4, hkv, d)), draw((4, hkv, d))
        q = draw((4, hq, d))
        out, slots = pool.decode_step(seqs, to_device(k, dtype), to_device(v, dtype), to_device(q, dtype))
        want_slots = []
        for i, s in enumerate(seqs):
            want_slots += ref.append(s, 1)
        assert slots.tolist() == want_slots
        ref.write(want_slots, to_f64(k, dtype), to_f64(v, dtype))
        got = to_host_f64(out)
        for i, s in enumerate(seqs):
            want = oracle.paged_attention(ref, s, to_f64(q[i:i + 1], dtype))[0]
            assert_close(got[i], want, *tol_, what=f"step {step} seq {s}")
    for s in seqs:
        assert pool.block_table(s).tolist() == ref.tables[s]
    assert [pool.refcount(b) for b in range(nb)] == ref.refs.tolist()


def test_decode_step_small_workspace_changes_nothing():
    from paged_kv_cache_block_amd.abi import InvalidArgumentError
    wl = _decode_case([10, 20], 8, 2, 64, 16)
    pool, _ = build_device_pool(wl)
    before = (pool.stats(), pool.block_table(0).tolist(), pool.seq_len(1))
    k = torch.zeros(2, 2, 64, dtype=torch.bfloat16, device="cuda")
    q = torch.zeros(2, 8, 64, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    from paged_kv_cache_block_amd import abi
    need = abi.pa_decode_step_workspace_bytes(pool.handle, [0, 1], 8)
    assert need >= 256
    with pytest.raises(InvalidArgumentError):
        abi.pa_decode_step(pool.handle, [0, 1], 8, k, k, q, torch.empty_like(q), ws, need - 1, None)
    assert before == (pool.stats(), pool.block_table(0).tolist(), pool.seq_len(1))


def test_copy_on_write_on_device():
    from paged_kv_cache_block_amd import DevicePool
    rng = np.random.default_rng(3)
    pool = DevicePool(16, 16, 2, 64, dtype="bf16", allocation_order=rng.permutation(16))
    k = torch.randn(21, 2, 64, dtype=torch.bfloat16, device="cuda")
    v = torch.randn(21, 2, 64, dtype=torch.bfloat16, device="cuda")
    pool.create(0)
    pool.write(pool.append(0, 21), k, v)
    pool.fork(0, 1)
    pool.fork(0, 2)
    s1 = pool.append(1, 1)             # COW of the shared partial tail
    s2 = pool.append(2, 2)             # another COW of the same source block
    assert len(pool.pending_copies()) == 2
    k1 = torch.randn(1, 2, 64, dtype=torch.bfloat16, device="cuda")
    k2 = torch.randn(2, 2, 64, dtype=torch.bfloat16, device="cuda")
    pool.write(s1, k1, k1)
    pool.write(s2, k2, k2)
    torch.cuda.synchronize()
    assert pool.pending_copies() == []
    K0, V0 = _gather_pool_rows(pool, 0, 21)
    K1, V1 = _gather_pool_rows(pool, 1, 22)
    K2, V2 = _gather_pool_rows(pool, 2, 23)
    np.testing.assert_array_equal(K1[:21], K0)
    np.testing.assert_array_equal(V2[:21], V0)
    np.testing.assert_array_equal(K1[21], k1[0].float().cpu().numpy())
    np.testing.assert_array_equal(K2[21:], k2.float().cpu().numpy())
    np.testing.assert_array_equal(K0, k.float().cpu().numpy())


# ------------------------------------------------------------ prefill
def test_prefix_prefill_small_full_compare():
    wl = prefix_prefill(batch=4, prefix=300, chunk=70, num_blocks=128, num_heads=32, num_kv_heads=8,
                        head_dim=128, block_size=16)
    log("prefill small: build")
    pool, ref = build_device_pool(wl, check_against_oracle_pool=True)
    assert pool.refcount(pool.block_table(0)[0]) == 4
    qp = prefill_queries(wl)
    seqs = [s for s, _ in wl.prefill]
    q_lens = [n for _, n in wl.prefill]
    out = to_host_f64(pool.prefill(seqs, q_lens, to_device(qp, wl.dtype)))
    rows = logical_kv(wl, seqs)
    r0 = 0
    for s, n in wl.prefill:
        K, V = (to_f64(x, wl.dtype) for x in rows[s])
        exp = oracle.attention(to_f64(qp[r0:r0 + n], wl.dtype), K, V)
        assert_close(out[r0:r0 + n], exp, *BF16_TOL, what=f"seq {s}")
        r0 += n


PREFILL_CASES = [
    # (kv lengths, q_lens), Hq, Hkv, D, bs
    (([600, 77, 40], [70, 77, 1]), 32, 8, 128, 16),     # GQA 4; no-prefix row; single row
    (([300, 129], [129, 33]), 64, 8, 128, 16),          # GQA 8
    (([200, 50], [31, 50]), 16, 16, 64, 32),            # MHA, D 64, bs 32
    (([333, 64], [100, 17]), 16, 1, 128, 32),           # GQA 16
    (([150, 90], [41, 90]), 8, 4, 64, 16),              # GQA 2
    (([120, 61], [19, 61]), 6, 2, 64, 16),              # GQA 3: generic kernel
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: f"G{c[1]//c[2]}-D{c[3]}-bs{c[4]}")
def test_prefill_shapes(case):
    (lengths, q_lens), hq, hkv, d, bs = case
    nb = int(sum(-(-n // bs) for n in lengths) + 5)
    order = np.random.default_rng(11).permutation(nb).astype(np.int32)
    ops = []
    for i, n in enumerate(lengths):
        ops += [("create", i), ("append", i, int(n))]
    wl = Workload("prefill_case", 9, "bf16", nb, bs, hq, hkv, d, order, ops,
                  prefill=[(i, q) for i, q in enumerate(q_lens)])
    log(f"prefill case {case}")
    pool, _ = build_device_pool(wl, check_against_oracle_pool=True)
    qp = prefill_queries(wl)
    out = to_host_f64(pool.prefill(list(range(len(lengths))), q_lens, to_device(qp, wl.dtype)))
    rows = logical_kv(wl, list(range(len(lengths))))
    r0 = 0
    for s, n in wl.prefill:
        K, V = (to_f64(x, wl.dtype) for x in rows[s])
        exp = oracle.attention(to_f64(qp[r0:r0 + n], wl.dtype), K, V)
        assert_close(out[r0:r0 + n], exp, *BF16_TOL, what=f"seq {s}")
        r0 += n


@pytest.mark.parametrize("shape", [(32, 8, 128, 16), (16, 16, 64, 32), (8, 2, 16, 4)],
                         ids=["G4-D128-bs16", "G1-D64-bs32", "generic"])
def test_unused_slots_holding_nan_do_not_leak(shape):
    """Slots past a sequence's end are never read into the result, even when
    the caller's pool memory holds NaN there."""
    from paged_kv_cache_block_amd import DevicePool
    hq, hkv, d, bs = shape
    lengths, q_lens = [37, 5, 70], [9, 5, 33]
    nb = sum(-(-n // bs) for n in lengths) + 3
    order = np.random.default_rng(2).permutation(nb).astype(np.int32)
    ops = []
    for i, n in enumerate(lengths):
        ops += [("create", i), ("append", i, n)]
    wl = Workload("nan_case", 12, "bf16", nb, bs, hq, hkv, d, order, ops,
                  decode_seqs=[0, 1, 2], prefill=[(i, q) for i, q in enumerate(q_lens)])
    pool = DevicePool(nb, bs, hkv, d, dtype="bf16", allocation_order=order)
    pool.k.fill_(float("nan"))
    pool.v.fill_(float("nan"))
    for op in append_stream(wl):
        if op[0] == "create":
            pool.create(op[1])
        elif op[0] == "append":
            _, s, n, k, v = op
            pool.write(pool.append(s, n), to_device(k, "bf16"), to_device(v, "bf16"))
    q_bits, got = _decode(pool, wl, [0, 1, 2])
    want = expected_decode(wl, [0, 1, 2], q_bits)
    for i in range(3):
        assert_close(got[i], want[i], *BF16_TOL, what=f"decode seq {i}")
    qp = prefill_queries(wl)
    out = to_host_f64(pool.prefill([0, 1, 2], q_lens, to_device(qp, "bf16")))
    rows = logical_kv(wl, [0, 1, 2])
    r0 = 0
    for s, n in wl.prefill:
        K, V = (to_f64(x, "bf16") for x in rows[s])
        assert_close(out[r0:r0 + n], oracle.attention(to_f64(qp[r0:r0 + n], "bf16"), K, V),
                     *BF16_TOL, what=f"prefill seq {s}")
        r0 += n


def test_prefill_rejects_bad_rows():
    from paged_kv_cache_block_amd.abi import InvalidArgumentError
    wl = _decode_case([10, 20], 8, 2, 64, 16)
    pool, _ = build_device_pool(wl)
    q = torch.zeros(21, 8, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(InvalidArgumentError):
        pool.prefill([0], [11], q[:11])         # 11 rows of a 10-token sequence
    with pytest.raises(InvalidArgumentError):
        pool.prefill([0, 1], [0, 5], q[:5])     # an empty chunk


# ------------------------------------------------------------ full size
def test_gqa_decode_full_size():
    wl = gqa_decode()
    log("gqa_decode full: build")
    pool, _ = build_device_pool(wl)
    st = pool.stats()
    assert st["allocated_blocks"] == 8183 and st["logical_tokens"] == 130736
    seqs = wl.decode_seqs
    log("gqa_decode full: decode")
    q_bits, got = _decode(pool, wl, seqs)
    log("gqa_decode full: oracle")
    want = expected_decode(wl, seqs, q_bits)
    for i in seqs:
        assert_close(got[i], want[i], *BF16_TOL, what=f"seq {i}")


def _expected_each(wl, seqs, q_bits, rows):
    """Oracle decode rows of ``seqs``, one sequence at a time (its rows
    widened to float64 and released before the next)."""
    for i, s in enumerate(seqs):
        K, V = rows[s]
        yield i, s, oracle.attention(to_f64(q_bits[i:i + 1], wl.dtype), to_f64(K, wl.dtype),
                                     to_f64(V, wl.dtype))[0]


def test_long_decode_full_size():
    """Every output of workload 3 (4 x 131,072 tokens, 64 / 8 heads): split-K
    over 32 page ranges per sequence and the log-sum-exp merge, in the launch
    configuration the bench times."""
    wl = long_decode()
    log("long_decode full: build")
    pool, rows = build_device_pool_keeping_rows(wl)
    assert pool.stats()["free_blocks"] == 0
    seqs = wl.decode_seqs
    q_bits, got = _decode(pool, wl, seqs)
    pool.close()
    for i, s, want in _expected_each(wl, seqs, q_bits, rows):
        log(f"long_decode full: oracle on sequence {s}")
        assert_close(got[i], want, *BF16_TOL, what=f"seq {s}")


def test_heavy_tail_full_size():
    """Every output of workload 5: 256 sequences of 17 .. 32,373 tokens, MHA
    d 64, bs 32, 1% of K/V rows x8 (the softmax maximum's stress case)."""
    wl = heavy_tail()
    log("heavy_tail full: build")
    pool, rows = build_device_pool_keeping_rows(wl)
    st = pool.stats()
    assert st["allocated_blocks"] == 42982 and st["logical_tokens"] == 1371446
    seqs = wl.decode_seqs
    q_bits, got = _decode(pool, wl, seqs)
    pool.close()
    lengths = wl.final_lengths()
    log(f"heavy_tail full: oracle on all {len(seqs)} sequences")
    for i, s, want in _expected_each(wl, seqs, q_bits, rows):
        assert_close(got[i], want, *BF16_TOL, what=f"seq {s} (L={lengths[s]})")
        if i % 64 == 63:
            log(f"heavy_tail full: {i + 1} sequences compared")


def test_prefix_prefill_full_size():
    """Every output row x head of workload 4: 16 x 512 causal rows over a
    4096-token prefix shared by all 16 sequences (refcount 16) plus their own
    512 tokens."""
    wl = prefix_prefill()
    log("prefix_prefill full: build")
    pool, rows = build_device_pool_keeping_rows(wl)
    st = pool.stats()
    assert st["allocated_blocks"] == 768 and pool.refcount(pool.block_table(0)[0]) == 16
    qp = prefill_queries(wl)
    seqs = [s for s, _ in wl.prefill]
    q_lens = [n for _, n in wl.prefill]
    log("prefix_prefill full: prefill")
    out = to_host_f64(pool.prefill(seqs, q_lens, to_device(qp, wl.dtype)))
    torch.cuda.synchronize()
    pool.close()
    r0 = 0
    for s, n in wl.prefill:
        K, V = (to_f64(x, wl.dtype) for x in rows[s])
        want = oracle.attention(to_f64(qp[r0:r0 + n], wl.dtype), K, V)
        assert_close(out[r0:r0 + n], want, *BF16_TOL, what=f"prefill seq {s}")
        r0 += n
    log(f"prefix_prefill full: {r0} rows x {wl.num_heads} heads compared")


@pytest.mark.parametrize("bs,d", [(16, 128), (32, 64), (16, 64), (8, 128), (16, 48), (128, 128)])
def test_bf16_pages_hold_rows_at_documented_places(bs, d):
    """pa_reshape_and_cache and the step prologue put every K value where the
    header's page order says (reordered tiles for bs % 16 == 0 and d % 32 ==
    0, row-major otherwise) and every V value at [d][slot]."""
    from paged_kv_cache_block_amd import DevicePool
    hkv, nb = 2, 12
    pool = DevicePool(nb, bs, hkv, d, dtype="bf16", allocation_order=np.random.default_rng(bs + d).permutation(nb))
    gen = torch.Generator(device="cuda").manual_seed(bs * d)
    n0 = 3 * bs + 5
    k = torch.randn(n0, hkv, d, generator=gen, device="cuda").to(torch.bfloat16)
    v = torch.randn(n0, hkv, d, generator=gen, device="cuda").to(torch.bfloat16)
    pool.create(0)
    pool.write(pool.append(0, n0), k, v)
    # One decode step appends and stores a row through the fused prologue.
    kn = torch.randn(1, hkv, d, generator=gen, device="cuda").to(torch.bfloat16)
    vn = torch.randn(1, hkv, d, generator=gen, device="cuda").to(torch.bfloat16)
    q = torch.randn(1, 2 * hkv, d, generator=gen, device="cuda").to(torch.bfloat16)
    pool.decode_step([0], kn, vn, q)
    torch.cuda.synchronize()
    K, V = _gather_pool_rows(pool, 0, n0 + 1)
    np.testing.assert_array_equal(K, torch.cat([k, kn]).float().cpu().numpy())
    np.testing.assert_array_equal(V, torch.cat([v, vn]).float().cpu().numpy())
