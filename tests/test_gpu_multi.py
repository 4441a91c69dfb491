"""GPU parity of multi-token queries (q_len 2..32 rows per sequence, the
last positions) on the split-K decode kernels: the fused verify step
(append + cache write + causal attention) and short prefill chunks.

Source: docs.rs ferrum-kv 0.4.0 src/attention.rs, paged_attention with
q_tokens > 1 (row t sees keys j <= kv_len - q_tokens + t).  Bar: slots,
tables and refcounts bit-exact; outputs within (2e-3, 1e-2) of the float64
oracle (int8 pages: of the oracle over the rows read back).
"""

import numpy as np
import pytest

import oracle
from synth import decode_queries, gqa_decode, logical_kv
from synth.workloads import bf16_round, to_f64

from gpu_support import BF16_TOL, assert_close, log, to_device, to_host_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_block_amd import abi
    abi.load()


def _setup(lengths, hq, hkv, d, bs, kv, seed=5, fork=True):
    from paged_kv_cache_block_amd import DevicePool
    nb = int(sum(-(-n // bs) for n in lengths) * 2 + 64)
    order = np.random.default_rng(seed).permutation(nb).astype(np.int32)
    pool = DevicePool(nb, bs, hkv, d, dtype=kv, allocation_order=order)
    ref = oracle.Pool(nb, bs, hkv, d, allocation_order=order, quant_bits=8 if kv in ("i8", "fp8") else None,
                     quant_fp8=kv == "fp8")
    rng = np.random.default_rng(seed + 1)
    for s, n in enumerate(lengths):
        pool.create(s)
        ref.create(s)
        k = bf16_round(rng.standard_normal((n, hkv, d)).astype(np.float32))
        v = bf16_round(rng.standard_normal((n, hkv, d)).astype(np.float32))
        slots = pool.append(s, n)
        assert slots.tolist() == ref.append(s, n)
        pool.write(slots, to_device(k, "bf16"), to_device(v, "bf16"))
        ref.write(slots, to_f64(k, "bf16"), to_f64(v, "bf16"))
    seqs = list(range(len(lengths)))
    if fork:
        # The fork shares sequence 1's partial tail: its first verify copies it.
        pool.fork(1, len(lengths))
        ref.fork(1, len(lengths))
        seqs.append(len(lengths))
    return pool, ref, rng, seqs


def _expected(ref, seqs, q_lens, q):
    out, r0 = [], 0
    for s, n in zip(seqs, q_lens):
        keys, values = ref.gather(s)
        out.append(oracle.attention(to_f64(q[r0:r0 + n], "bf16"), keys, values))
        r0 += n
    return np.concatenate(out)


VERIFY_CASES = [
    # lengths, q_lens (the fork last), Hq, Hkv, D, bs, kv
    ([1, 15, 33, 700, 5000], [1, 2, 4, 8, 5, 3], 32, 8, 128, 16, "bf16"),   # G4: 32 columns
    ([9, 300, 4100, 64], [1, 4, 3, 2, 4], 64, 8, 128, 16, "bf16"),          # G8
    ([5, 40, 2049], [16, 32, 1, 7], 16, 16, 64, 32, "bf16"),                 # MHA, 32 rows
    ([3, 77, 3000], [4, 8, 1, 2], 32, 8, 128, 16, "i8"),                     # int8 pages
    ([20, 513], [16, 3, 9], 8, 4, 64, 16, "i8"),                             # int8, G2, D64
    ([3, 77, 3000], [4, 8, 1, 2], 32, 8, 128, 16, "fp8"),                    # E4M3 pages
    ([20, 513], [16, 3, 9], 8, 4, 64, 16, "fp8"),                            # E4M3, G2, D64
    ([31, 1000], [2, 3, 4], 16, 2, 128, 32, "bf16"),                         # G8, bs 32
]


@pytest.mark.parametrize("case", VERIFY_CASES,
                         ids=lambda c: f"G{c[2]//c[3]}-D{c[4]}-bs{c[5]}-{c[6]}-q{max(c[1])}")
def test_verify_step_matches_oracle(case):
    lengths, q_lens, hq, hkv, d, bs, kv = case
    log(f"verify {case}")
    pool, ref, rng, seqs = _setup(lengths, hq, hkv, d, bs, kv)
    assert len(seqs) == len(q_lens)
    for step in range(3):
        ql = [max(1, q - step) for q in q_lens]
        rows = sum(ql)
        k = bf16_round(rng.standard_normal((rows, hkv, d)).astype(np.float32))
        v = bf16_round(rng.standard_normal((rows, hkv, d)).astype(np.float32))
        q = bf16_round(rng.standard_normal((rows, hq, d)).astype(np.float32))
        out, slots = pool.verify_step(seqs, ql, to_device(k, "bf16"), to_device(v, "bf16"), to_device(q, "bf16"))
        want_slots = []
        for s, n in zip(seqs, ql):
            want_slots += ref.append(s, n)
        assert slots.tolist() == want_slots
        ref.write(want_slots, to_f64(k, "bf16"), to_f64(v, "bf16"))
        got = to_host_f64(out)
        want = _expected(ref, seqs, ql, q)
        assert_close(got, want, *BF16_TOL, what=f"step {step}")
    for s in seqs:
        assert pool.block_table(s).tolist() == ref.tables[s]
    assert [pool.refcount(b) for b in range(ref.num_blocks)] == ref.refs.tolist()
    pool.validate()


def test_verify_step_rejections_change_nothing():
    from paged_kv_cache_block_amd import DevicePool
    from paged_kv_cache_block_amd.abi import InvalidArgumentError
    pool, ref, rng, seqs = _setup([40, 50], 32, 8, 128, 16, "bf16", fork=False)
    k = torch.zeros(64, 8, 128, dtype=torch.bfloat16, device="cuda")
    q = torch.zeros(64, 32, 128, dtype=torch.bfloat16, device="cuda")
    before = (pool.stats(), pool.block_table(0).tolist(), pool.seq_len(1))
    for s_, ql in (([0, 0], [1, 1]),        # a sequence twice
                   ([0, 1], [9, 1]),        # 9 rows x G 4 = 36 columns
                   ([0, 1], [0, 1])):       # empty row set
        with pytest.raises(InvalidArgumentError):
            pool.verify_step(s_, ql, k[:sum(ql)], k[:sum(ql)], q[:sum(ql)])
    assert before == (pool.stats(), pool.block_table(0).tolist(), pool.seq_len(1))
    f32 = DevicePool(16, 16, 2, 64, dtype="f32")
    f32.create(0)
    f32.append(0, 3)
    with pytest.raises(InvalidArgumentError):
        f32.verify_step([0], [2], torch.zeros(2, 2, 64, device="cuda"), torch.zeros(2, 2, 64, device="cuda"),
                        torch.zeros(2, 4, 64, device="cuda"))
    assert f32.seq_len(0) == 3


@pytest.mark.parametrize("kv", ["bf16", "i8", "fp8"])
def test_short_prefill_chunks_use_split_k(kv):
    """pa_prefill_chunk with every q_len * G <= 32 runs on the decode
    kernels (rows of a split sequence merge by log-sum-exp)."""
    lengths, q_lens = [600, 77, 8, 4100], [3, 8, 8, 5]
    pool, ref, rng, seqs = _setup(lengths, 32, 8, 128, 16, kv, fork=False)
    q = bf16_round(rng.standard_normal((sum(q_lens), 32, 128)).astype(np.float32))
    got = to_host_f64(pool.prefill(seqs, q_lens, to_device(q, "bf16")))
    assert_close(got, _expected(ref, seqs, q_lens, q), *BF16_TOL, what="short prefill")


def test_verify_full_size_sampled():
    """gqa_decode (32 x U[1, 8192], 32/8 heads, d 128, bs 16) with 4 query
    rows per sequence (3 drafted tokens + 1): sampled sequences."""
    from paged_kv_cache_block_amd import DevicePool
    from synth import append_stream
    wl = gqa_decode()
    log("verify full size: build")
    pool = DevicePool(wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim, dtype="bf16",
                      allocation_order=wl.allocation_order)
    for op in append_stream(wl):
        if op[0] == "create":
            pool.create(op[1])
        else:
            _, s, n, k, v = op
            pool.write(pool.append(s, n), to_device(k, "bf16"), to_device(v, "bf16"))
    seqs = list(wl.decode_seqs)
    q_lens = [4] * len(seqs)
    rng = np.random.default_rng(99)
    rows = 4 * len(seqs)
    k_new = bf16_round(rng.standard_normal((rows, 8, 128)).astype(np.float32))
    v_new = bf16_round(rng.standard_normal((rows, 8, 128)).astype(np.float32))
    q = bf16_round(rng.standard_normal((rows, 32, 128)).astype(np.float32))
    log("verify full size: step")
    out, _ = pool.verify_step(seqs, q_lens, to_device(k_new, "bf16"), to_device(v_new, "bf16"), to_device(q, "bf16"))
    got = to_host_f64(out)
    lengths = wl.final_lengths()
    sample = sorted({int(np.argmax([lengths[s] for s in seqs])), int(np.argmin([lengths[s] for s in seqs])), 5, 21})
    rows_kv = logical_kv(wl, sample)
    for s in sample:
        K = np.concatenate([to_f64(rows_kv[s][0], "bf16"), to_f64(k_new[4 * s:4 * s + 4], "bf16")])
        V = np.concatenate([to_f64(rows_kv[s][1], "bf16"), to_f64(v_new[4 * s:4 * s + 4], "bf16")])
        want = oracle.attention(to_f64(q[4 * s:4 * s + 4], "bf16"), K, V)
        assert_close(got[4 * s:4 * s + 4], want, *BF16_TOL, what=f"seq {s} (L={K.shape[0]})")
