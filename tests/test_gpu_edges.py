"""GPU parity at the edges of the supported shapes: the largest head_dim
(512), large and tiny blocks, a single slot per block, group 16 and a
single query head per KV head, 8-bit pages on the generic kernel (head_dim
256), one-token sequences, a batch of one, chunks whose rows reach the
first position of the sequence, pools larger than 4 GiB, and the debug slot
checks of the cache writes.

Source: docs.rs ferrum-kv 0.4.0 src/attention.rs, paged_attention (decode and
q_tokens > 1); int8 rows as in the vladkulikov.com notebook "Модуль 10"
KV-compression experiment.  Bar: (1e-5, 1e-5) fp32, (2e-3, 1e-2) bf16 / int8.
"""

import numpy as np
import pytest

import oracle
from synth.workloads import bf16_round, to_f64

from gpu_support import BF16_TOL, F32_TOL, assert_close, log, to_device, to_host_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_block_amd import abi
    abi.load()


def _io(kv):
    return "f32" if kv == "f32" else "bf16"


def _draw(rng, shape, kv):
    x = rng.standard_normal(shape).astype(np.float32)
    return x if kv == "f32" else bf16_round(x)


def _pool(lengths, hkv, d, bs, kv, seed=1):
    from paged_kv_cache_block_amd import DevicePool
    nb = int(sum(-(-n // bs) for n in lengths) + 5)
    order = np.random.default_rng(seed).permutation(nb).astype(np.int32)
    pool = DevicePool(nb, bs, hkv, d, dtype=kv, allocation_order=order)
    ref = oracle.Pool(nb, bs, hkv, d, allocation_order=order, quant_bits=8 if kv in ("i8", "fp8") else None,
                     quant_fp8=kv == "fp8")
    rng = np.random.default_rng(seed + 7)
    io = _io(kv)
    for s, n in enumerate(lengths):
        pool.create(s)
        ref.create(s)
        k, v = _draw(rng, (n, hkv, d), kv), _draw(rng, (n, hkv, d), kv)
        slots = pool.append(s, n)
        assert slots.tolist() == ref.append(s, n)
        pool.write(slots, to_device(k, io), to_device(v, io))
        ref.write(slots, to_f64(k, io), to_f64(v, io))
    torch.cuda.synchronize()
    return pool, ref, rng


EDGE_CASES = [
    # lengths, Hq, Hkv, D, bs, kv
    ([1, 3, 700], 4, 2, 512, 16, "f32"),        # largest head_dim, generic fp32
    ([2, 65, 300], 8, 4, 512, 8, "bf16"),       # largest head_dim, bf16 generic
    ([1, 129, 1000], 8, 1, 64, 1, "f32"),       # one slot per block
    ([5, 300, 2000], 8, 8, 128, 128, "bf16"),   # large block (generic), MHA
    ([1, 2, 17, 900], 16, 1, 128, 16, "bf16"),  # group 16 on the MFMA kernel
    ([1, 40, 1200], 16, 2, 256, 32, "i8"),      # int8 pages, head_dim 256 (generic)
    ([7], 32, 8, 128, 16, "bf16"),              # a batch of one
    ([1, 1, 1], 32, 8, 128, 16, "i8"),          # one-token sequences, int8
    ([1, 40, 1200], 16, 2, 256, 32, "fp8"),     # E4M3 pages, head_dim 256 (generic)
    ([1, 1, 1], 32, 8, 128, 16, "fp8"),         # one-token sequences, E4M3
]


@pytest.mark.parametrize("case", EDGE_CASES,
                         ids=lambda c: f"D{c[3]}-bs{c[4]}-G{c[1]//c[2]}-{c[5]}-L{max(c[0])}")
def test_decode_and_prefill_edges(case):
    lengths, hq, hkv, d, bs, kv = case
    log(f"edge {case}")
    pool, ref, rng = _pool(lengths, hkv, d, bs, kv)
    io = _io(kv)
    tol = F32_TOL if kv == "f32" else BF16_TOL
    seqs = list(range(len(lengths)))
    q = _draw(rng, (len(seqs), hq, d), io)
    got = to_host_f64(pool.decode(seqs, to_device(q, io)))
    for i, s in enumerate(seqs):
        want = oracle.paged_attention(ref, s, to_f64(q[i:i + 1], io))[0]
        assert_close(got[i], want, *tol, what=f"decode seq {s}")
    # Prefill: every row of each sequence (rows reach position 0).
    q_lens = list(lengths)
    qp = _draw(rng, (sum(q_lens), hq, d), io)
    got = to_host_f64(pool.prefill(seqs, q_lens, to_device(qp, io)))
    r0 = 0
    for s, n in zip(seqs, q_lens):
        keys, values = ref.gather(s)
        want = oracle.attention(to_f64(qp[r0:r0 + n], io), keys, values)
        assert_close(got[r0:r0 + n], want, *tol, what=f"prefill seq {s}")
        r0 += n


def test_reshape_and_cache_skips_out_of_range_slots():
    """Slots outside [0, num_blocks * block_size) are skipped (documented):
    the pool bytes do not change."""
    from paged_kv_cache_block_amd import DevicePool
    pool = DevicePool(4, 16, 2, 64, dtype="bf16")
    before = pool.k.clone(), pool.v.clone()
    k = torch.ones(3, 2, 64, dtype=torch.bfloat16, device="cuda")
    slots = torch.tensor([-1, 64, 1 << 40], dtype=torch.int64, device="cuda")
    pool.write(slots, k, k)
    torch.cuda.synchronize()
    assert torch.equal(pool.k, before[0]) and torch.equal(pool.v, before[1])
    for kind in ("i8", "fp8"):
        q8 = DevicePool(4, 16, 2, 64, dtype=kind)
        before = q8.k.clone()
        q8.write(slots, k, k)
        torch.cuda.synchronize()
        assert torch.equal(q8.k, before)


@pytest.mark.parametrize("kv", ["bf16", "i8"])
def test_slot_checks_reject_bad_slots_before_writing(kv):
    """With slot checks on, a slot outside the pool or a slot two rows of one
    call name is rejected with PA_ERR_INVALID_ARG and nothing is written
    (the [PagedPool] negative tests' rule: validate before mutate); valid
    rows are then stored as usual, pending copy-on-write copies included, and
    a second valid call with the same slots passes (stamps differ per call)."""
    from paged_kv_cache_block_amd import DevicePool
    from paged_kv_cache_block_amd.abi import InvalidArgumentError
    pool = DevicePool(8, 16, 2, 64, dtype=kv)
    pool.set_slot_checks(True)
    pool.create(0)
    pool.append(0, 20)
    pool.fork(0, 1)
    slots = pool.append(1, 3)  # copy-on-write of the shared partial tail, left pending
    assert pool.pending_copies()
    torch.cuda.synchronize()
    before = pool.k.clone(), pool.v.clone()
    rows = torch.ones(3, 2, 64, dtype=torch.bfloat16, device="cuda")
    log(f"slot checks ({kv}): out of range")
    for bad in ([int(slots[0]), 8 * 16, int(slots[2])], [-1, int(slots[1]), int(slots[2])]):
        with pytest.raises(InvalidArgumentError, match="outside"):
            pool.write(torch.tensor(bad, dtype=torch.int64, device="cuda"), rows, rows)
    log(f"slot checks ({kv}): repeated slot")
    with pytest.raises(InvalidArgumentError, match="also names"):
        pool.write(torch.tensor([int(slots[0]), int(slots[1]), int(slots[0])], dtype=torch.int64,
                                device="cuda"), rows, rows)
    torch.cuda.synchronize()
    assert torch.equal(pool.k, before[0]) and torch.equal(pool.v, before[1])
    assert pool.pending_copies(), "a rejected call must not flush the pending copies"
    log(f"slot checks ({kv}): valid rows, twice")
    good = torch.as_tensor(slots, dtype=torch.int64).cuda()
    pool.write(good, rows, rows)
    pool.write(good, rows, rows)
    torch.cuda.synchronize()
    assert not pool.pending_copies()
    assert not torch.equal(pool.k, before[0])
    pool.set_slot_checks(False)
    pool.validate()
    pool.close()


@pytest.mark.parametrize("kv", ["bf16", "i8"])
def test_pools_beyond_4_gib(kv):
    """Each pool larger than 4 GiB, its highest blocks handed out first, so
    every page address needs more than 32 bits: cache writes, a decode step,
    decode and prefill read the rows back within tolerance of the oracle
    (attention over the rows as written, or as read back for int8)."""
    from paged_kv_cache_block_amd import DevicePool, abi
    hq, hkv, d, bs = 32, 8, 128, 16
    page = bs * d * 2 if kv == "bf16" else bs * d + 4 * bs
    nb = (4 << 30) // (hkv * page) + 4096
    assert abi.pa_pool_bytes(abi.make_desc(nb, bs, hkv, d, abi.PA_DTYPE_BF16 if kv == "bf16" else abi.PA_DTYPE_I8)) > 4 << 30
    order = np.arange(nb - 1, -1, -1, dtype=np.int32)      # highest block first
    log(f"pool beyond 4 GiB ({kv}): {nb} blocks")
    pool = DevicePool(nb, bs, hkv, d, dtype=kv, allocation_order=order)
    rng = np.random.default_rng(44)
    lengths = [37, 300, 1000]
    rows = []
    for s, n in enumerate(lengths):
        pool.create(s)
        k, v = bf16_round(rng.standard_normal((n, hkv, d)).astype(np.float32)), \
            bf16_round(rng.standard_normal((n, hkv, d)).astype(np.float32))
        slots = pool.append(s, n)
        assert int(slots.min()) >= (nb - 100) * bs
        pool.write(slots, to_device(k, "bf16"), to_device(v, "bf16"))
        rows.append([to_f64(k, "bf16"), to_f64(v, "bf16")])
    kn = bf16_round(rng.standard_normal((3, hkv, d)).astype(np.float32))
    vn = bf16_round(rng.standard_normal((3, hkv, d)).astype(np.float32))
    q = bf16_round(rng.standard_normal((3, hq, d)).astype(np.float32))
    out, _ = pool.decode_step([0, 1, 2], to_device(kn, "bf16"), to_device(vn, "bf16"), to_device(q, "bf16"))
    for s in range(3):
        rows[s][0] = np.concatenate([rows[s][0], to_f64(kn[s:s + 1], "bf16")])
        rows[s][1] = np.concatenate([rows[s][1], to_f64(vn[s:s + 1], "bf16")])

    def kv_of(s):
        K, V = rows[s]
        if kv == "i8":
            return oracle.fake_quantize_rows(K, 8), oracle.fake_quantize_rows(V, 8)
        return K, V

    got = to_host_f64(out)
    for s in range(3):
        K, V = kv_of(s)
        assert_close(got[s], oracle.attention(to_f64(q[s:s + 1], "bf16"), K, V)[0], *BF16_TOL,
                     what=f"decode step seq {s}")
    q_lens = [37, 64, 200]
    qp = bf16_round(rng.standard_normal((sum(q_lens), hq, d)).astype(np.float32))
    outp = to_host_f64(pool.prefill([0, 1, 2], q_lens, to_device(qp, "bf16")))
    r0 = 0
    for s, n in enumerate(q_lens):
        K, V = kv_of(s)
        assert_close(outp[r0:r0 + n], oracle.attention(to_f64(qp[r0:r0 + n], "bf16"), K, V), *BF16_TOL,
                     what=f"prefill seq {s}")
        r0 += n
    pool.close()
    del pool
    torch.cuda.empty_cache()


def test_binding_rejects_mismatched_tensors():
    """The Python binding checks every tensor it hands to the library (the
    kernels trust the pointers): wrong row counts, head_dim, dtype, device or
    layout raise ValueError before any call, and the pool is unchanged."""
    from paged_kv_cache_block_amd import DevicePool
    pool = DevicePool(16, 16, 2, 64, dtype="bf16")
    pool.create(0)
    pool.create(1)
    k = torch.zeros(10, 2, 64, dtype=torch.bfloat16, device="cuda")
    pool.write(pool.append(0, 10), k, k)
    pool.write(pool.append(1, 10), k, k)
    torch.cuda.synchronize()
    q = torch.zeros(2, 8, 64, dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros(2, 2, 64, dtype=torch.bfloat16, device="cuda")
    bad_q = [torch.zeros(3, 8, 64, dtype=torch.bfloat16, device="cuda"),       # rows
             torch.zeros(2, 8, 32, dtype=torch.bfloat16, device="cuda"),       # head_dim
             torch.zeros(2, 8, 64, dtype=torch.float32, device="cuda"),        # dtype
             torch.zeros(2, 8, 64, dtype=torch.bfloat16),                      # host memory
             torch.zeros(2, 64, 8, dtype=torch.bfloat16, device="cuda").transpose(1, 2)]  # layout
    for bq in bad_q:
        with pytest.raises(ValueError):
            pool.decode([0, 1], bq)
        with pytest.raises(ValueError):
            pool.decode_step([0, 1], kn, kn, bq)
    with pytest.raises(ValueError):
        pool.decode([0, 1], q, out=torch.zeros(1, 8, 64, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        pool.decode_step([0, 1], kn[:1], kn, q)
    with pytest.raises(ValueError):
        pool.verify_step([0, 1], [2, 1], kn, kn, q)           # 3 rows, tensors of 2
    with pytest.raises(ValueError):
        pool.prefill([0, 1], [2, 2], q)                       # 4 rows, q of 2
    with pytest.raises(ValueError):
        pool.write(np.zeros(0, dtype=np.int64), kn, kn)       # 0 slots, 2 rows
    assert pool.seq_len(0) == 10 and pool.seq_len(1) == 10
    out = pool.decode([0, 1], q)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
