"""GPU parity of 8-bit KV pages (codes + one fp32 scale per (token, KV head)
row) against the oracle's quantised pool, for both code kinds: int8
("i8") and 8-bit floats E4M3 ("fp8").

Source of the quantisation: vladkulikov.com notebook "Модуль 10", the
KV-compression experiment (integer codes); the 8-bit float codes keep its
per-row absmax scheme with E4M3 values (a reading beyond the pages).  The
oracle (oracle.quant, oracle.fp8) decides codes in float64 and keeps the
scale as fp32, and so do the cache-write kernels.

Bar: codes and scales written by the cache kernels are bit-exact against the
oracle; attention over 8-bit pages is within the bf16 tolerance (2e-3, 1e-2)
of the float64 oracle attention over the rows read back (value * scale).
"""

import numpy as np
import pytest

import oracle
from synth import append_stream, decode_queries, gqa_decode, logical_kv, prefill_queries, prefix_prefill
from synth.workloads import Workload, bf16_round, to_f64

from gpu_support import BF16_TOL, assert_close, k8_index, log, to_device, to_host_f64, v8_index

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_block_amd import abi
    abi.load()


KINDS = ["i8", "fp8"]


# ------------------------------------------------------------ helpers
def _device_codes(pool):
    """(K codes, K scales, V codes, V scales) of the whole device pool, in the
    oracle's [block][slot][head][dim] order (views where possible); int8
    codes signed, E4M3 codes as bytes (the oracle's code numbering)."""
    bs, d = pool.block_size, pool.head_dim
    code_t = np.uint8 if pool.dtype == "fp8" else np.int8

    def split(raw):
        codes = np.ascontiguousarray(raw[..., :bs * d]).view(code_t)      # [N, Hkv, bs*D]
        scales = np.ascontiguousarray(raw[..., bs * d:]).view(np.float32)  # [N, Hkv, bs]
        return codes, scales.transpose(0, 2, 1)

    kcodes, kscales = split(pool.k.cpu().numpy())
    vcodes, vscales = split(pool.v.cpu().numpy())
    kc = kcodes[..., k8_index(bs, d)].transpose(0, 2, 1, 3)
    vc = vcodes[..., v8_index(bs, d)].transpose(0, 2, 1, 3)
    return kc, kscales, vc, vscales


def _oracle_pool(nb, bs, hkv, d, order, kind):
    return oracle.Pool(nb, bs, hkv, d, allocation_order=order, quant_bits=8, quant_fp8=kind == "fp8")


def _fake_quant(x, kind):
    return oracle.fake_quantize_rows_fp8(x) if kind == "fp8" else oracle.fake_quantize_rows(x, 8)


def _quant(x, kind):
    return oracle.quantize_rows_fp8(x) if kind == "fp8" else oracle.quantize_rows(x, 8)


def _replay(wl, kind, mirror=True):
    """Build a DevicePool of ``kind`` from ``wl``'s op list and (``mirror``)
    the oracle's quantised pool from the same rows."""
    from paged_kv_cache_block_amd import DevicePool
    pool = DevicePool(wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim, dtype=kind,
                      allocation_order=wl.allocation_order)
    ref = _oracle_pool(wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim,
                       wl.allocation_order, kind) if mirror else None
    for op in append_stream(wl):
        if op[0] == "create":
            pool.create(op[1])
            if ref:
                ref.create(op[1])
        elif op[0] == "share":
            pool.share(*op[1:])
            if ref:
                ref.share(*op[1:])
        else:
            _, s, n, k, v = op
            slots = pool.append(s, n)
            pool.write(slots, to_device(k, "bf16"), to_device(v, "bf16"))
            if ref:
                assert slots.tolist() == ref.append(s, n)
                ref.write(slots, to_f64(k, "bf16"), to_f64(v, "bf16"))
    torch.cuda.synchronize()
    return pool, ref


def _case(lengths, hq, hkv, d, bs, seed=5):
    nb = int(sum(-(-n // bs) for n in lengths) + 7)
    order = np.random.default_rng(seed).permutation(nb).astype(np.int32)
    ops = []
    for i, n in enumerate(lengths):
        ops += [("create", i), ("append", i, int(n))]
    return Workload("q8_case", seed, "bf16", nb, bs, hq, hkv, d, order, ops,
                    decode_seqs=list(range(len(lengths))))


def _check_codes(pool, ref, seqs):
    kc, ks, vc, vs = _device_codes(pool)
    for s in seqs:
        n = ref.lengths[s]
        blk = np.asarray(ref.tables[s])[np.arange(n) // ref.block_size]
        off = np.arange(n) % ref.block_size
        np.testing.assert_array_equal(kc[blk, off], ref.Kc[blk, off], err_msg=f"K codes of seq {s}")
        np.testing.assert_array_equal(vc[blk, off], ref.Vc[blk, off], err_msg=f"V codes of seq {s}")
        np.testing.assert_array_equal(ks[blk, off], ref.Ks[blk, off].astype(np.float32))
        np.testing.assert_array_equal(vs[blk, off], ref.Vs[blk, off].astype(np.float32))


# ------------------------------------------------------------ cache writes
@pytest.mark.parametrize("kind", KINDS)
def test_q8_cache_write_codes_and_scales_bit_exact(kind):
    wl = _case([1, 15, 16, 17, 200], 32, 8, 128, 16)
    log(f"q8 codes {kind}: build")
    pool, ref = _replay(wl, kind)
    # Rows with zeros (scale 1), ties and extremes.  int8: whole-number bf16
    # values with absmax 127 make x / scale exact, so half-way codes occur.
    # E4M3: absmax 448 gives scale 1; 17 and 19 lie half-way between the
    # neighbours 16, 18 and 18, 20 (ties to the even mantissa: 16 and 20),
    # 2^-10 and 3 * 2^-10 half-way between subnormals (to 0 and 2 * 2^-9).
    pool.create(9)
    ref.create(9)
    top = 448.0 if kind == "fp8" else 127.0
    rows = np.zeros((3, 8, 128), np.float32)
    rows[1] = np.linspace(-top, top, 128, dtype=np.float32)[None, :]
    if kind == "fp8":
        rows[2, :, :5] = [448.0, -17.0, 19.0, 2.0 ** -10, 3 * 2.0 ** -10]
    else:
        rows[2, :, :4] = [127.0, -63.5, 0.5, 2.5]
    k = bf16_round(rows)
    v = bf16_round(rows[::-1].copy())
    slots = pool.append(9, 3)
    assert slots.tolist() == ref.append(9, 3)
    pool.write(slots, to_device(k, "bf16"), to_device(v, "bf16"))
    ref.write(slots, to_f64(k, "bf16"), to_f64(v, "bf16"))
    torch.cuda.synchronize()
    assert ref.Ks[slots[0] // 16, slots[0] % 16].tolist() == [1.0] * 8
    if kind == "fp8":
        assert ref.Ks[slots[2] // 16, slots[2] % 16].tolist() == [1.0] * 8
        assert ref.Kc[slots[2] // 16, slots[2] % 16, 0, :5].tolist() == [0x7E, 0xD8, 0x5A, 0x00, 0x02]
    else:
        assert ref.Kc[slots[2] // 16, slots[2] % 16, 0, :4].tolist() == [127, -64, 0, 2]
    _check_codes(pool, ref, [0, 1, 2, 3, 4, 9])


@pytest.mark.parametrize("kind", KINDS)
def test_q8_pool_bytes_and_copy_on_write(kind):
    from paged_kv_cache_block_amd import DevicePool, abi
    for dt in (abi.PA_DTYPE_I8, abi.PA_DTYPE_FP8):
        assert abi.pa_pool_bytes(abi.make_desc(10, 16, 2, 64, dt)) == 10 * 2 * (16 * 64 + 64)
    rng = np.random.default_rng(3)
    pool = DevicePool(16, 16, 2, 64, dtype=kind, allocation_order=rng.permutation(16))
    k = torch.randn(21, 2, 64, dtype=torch.bfloat16, device="cuda")
    pool.create(0)
    pool.write(pool.append(0, 21), k, -k)
    pool.fork(0, 1)
    s1 = pool.append(1, 1)             # COW of the shared partial tail (5 live rows)
    (src, dst), = pool.pending_copies()
    src_bytes = pool.k[src].clone(), pool.v[src].clone()
    pool.write(s1, k[:1], k[:1])
    torch.cuda.synchronize()
    assert pool.pending_copies() == []
    kc, ks, vc, vs = _device_codes(pool)
    for a in (kc, ks, vc, vs):
        np.testing.assert_array_equal(a[dst, :5], a[src, :5])
    assert torch.equal(pool.k[src], src_bytes[0]) and torch.equal(pool.v[src], src_bytes[1])


# ------------------------------------------------------------ decode
Q8_DECODE_CASES = [
    # lengths, Hq, Hkv, D, bs
    ([1, 2, 15, 16, 17, 33, 200, 700], 32, 8, 128, 16),     # GQA 4, ragged tails
    ([1, 64, 129, 1000, 4100], 64, 8, 128, 16),             # GQA 8, split-K
    ([5, 31, 32, 33, 517, 2049], 16, 16, 64, 32),            # MHA, D 64, bs 32
    ([3, 100, 1500], 16, 1, 128, 16),                        # GQA 16
    ([9, 300, 3000], 16, 2, 128, 32),                        # GQA 8, bs 32
    ([7, 77, 777], 8, 4, 64, 16),                            # GQA 2, D 64
    ([2, 90, 1200], 6, 2, 32, 16),                           # generic kernel (D 32)
]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("case", Q8_DECODE_CASES, ids=lambda c: f"L{max(c[0])}-G{c[1]//c[2]}-D{c[3]}-bs{c[4]}")
def test_q8_decode_shapes(case, kind):
    lengths, hq, hkv, d, bs = case
    wl = _case(lengths, hq, hkv, d, bs)
    log(f"q8 decode {kind} {case}: build")
    pool, ref = _replay(wl, kind)
    seqs = list(range(len(lengths)))
    q_bits = decode_queries(wl, seqs)
    got = to_host_f64(pool.decode(seqs, to_device(q_bits, "bf16")))
    for i in seqs:
        want = oracle.paged_attention(ref, i, to_f64(q_bits[i:i + 1], "bf16"))[0]
        assert_close(got[i], want, *BF16_TOL, what=f"seq {i} (L={lengths[i]})")


@pytest.mark.parametrize("kind", KINDS)
def test_q8_unused_slots_hold_garbage(kind):
    """Unused slots of a tail page may hold any bytes (NaN scales included,
    and for E4M3 the not-a-number codes 0x7F / 0xFF in K and V): they take
    no part in the result, in decode and in prefill."""
    wl = _case([17, 33, 250], 32, 8, 128, 16)
    pool, ref = _replay(wl, kind, mirror=True)
    q_bits = decode_queries(wl, [0, 1, 2])
    want = [oracle.paged_attention(ref, i, to_f64(q_bits[i:i + 1], "bf16"))[0] for i in range(3)]
    q_lens = [17, 20, 100]
    qp = bf16_round(np.random.default_rng(4).standard_normal((sum(q_lens), 32, 128)).astype(np.float32))
    want_p = []
    for s, n in enumerate(q_lens):
        keys, values = ref.gather(s)
        r0 = sum(q_lens[:s])
        want_p.append(oracle.attention(to_f64(qp[r0:r0 + n], "bf16"), keys, values))
    bs, d = 16, 128
    for s in range(3):
        n = ref.lengths[s]
        blk = ref.tables[s][-1]
        for raw in (pool.k, pool.v):
            raw[blk, :, bs * d:].view(torch.float32)[:, n % bs:] = float("nan")
        # K codes of the past-end slots (for E4M3 not-a-number), and for
        # E4M3 the V codes too, at their documented bytes.
        pool.k[blk, :, torch.as_tensor(k8_index(bs, d)[n % bs:].ravel(), device="cuda")] = 0x7F
        if kind == "fp8":
            pool.v[blk, :, torch.as_tensor(v8_index(bs, d)[n % bs:].ravel(), device="cuda")] = 0xFF
    got = to_host_f64(pool.decode([0, 1, 2], to_device(q_bits, "bf16")))
    for i in range(3):
        assert_close(got[i], want[i], *BF16_TOL, what=f"decode seq {i}")
    out = to_host_f64(pool.prefill([0, 1, 2], q_lens, to_device(qp, "bf16")))
    r0 = 0
    for s, n in enumerate(q_lens):
        assert_close(out[r0:r0 + n], want_p[s], *BF16_TOL, what=f"prefill seq {s}")
        r0 += n


@pytest.mark.parametrize("kind", KINDS)
def test_q8_decode_step_with_fork(kind):
    from paged_kv_cache_block_amd import DevicePool
    hq, hkv, d, bs, nb = 32, 8, 128, 16, 128
    order = np.random.default_rng(21).permutation(nb).astype(np.int32)
    pool = DevicePool(nb, bs, hkv, d, dtype=kind, allocation_order=order)
    ref = _oracle_pool(nb, bs, hkv, d, order, kind)
    rng = np.random.default_rng(5)

    def draw(shape_):
        return bf16_round(rng.standard_normal(shape_).astype(np.float32))

    for s, n in enumerate([37, 15, 200]):
        pool.create(s)
        ref.create(s)
        k, v = draw((n, hkv, d)), draw((n, hkv, d))
        slots = pool.append(s, n)
        assert slots.tolist() == ref.append(s, n)
        pool.write(slots, to_device(k, "bf16"), to_device(v, "bf16"))
        ref.write(slots, to_f64(k, "bf16"), to_f64(v, "bf16"))
    pool.fork(0, 3)
    ref.fork(0, 3)
    seqs = [0, 1, 2, 3]
    for step in range(5):
        k, v, q = draw((4, hkv, d)), draw((4, hkv, d)), draw((4, hq, d))
        out, slots = pool.decode_step(seqs, to_device(k, "bf16"), to_device(v, "bf16"), to_device(q, "bf16"))
        want_slots = []
        for s in seqs:
            want_slots += ref.append(s, 1)
        assert slots.tolist() == want_slots
        ref.write(want_slots, to_f64(k, "bf16"), to_f64(v, "bf16"))
        got = to_host_f64(out)
        for i, s in enumerate(seqs):
            want = oracle.paged_attention(ref, s, to_f64(q[i:i + 1], "bf16"))[0]
            assert_close(got[i], want, *BF16_TOL, what=f"step {step} seq {s}")
    torch.cuda.synchronize()
    _check_codes(pool, ref, seqs)


# ------------------------------------------------------------ prefill
@pytest.mark.parametrize("case", [(([300, 77], [70, 77]), 32, 8, 128, 16),
                                  (([200, 50], [31, 1]), 16, 16, 64, 32),
                                  (([1000, 513, 33], [300, 513, 33]), 32, 4, 128, 32),
                                  (([700, 129, 16], [257, 129, 16]), 8, 4, 64, 16),
                                  (([500, 97], [100, 97]), 16, 16, 64, 32),
                                  (([64, 65, 95], [64, 33, 95]), 16, 1, 128, 16)],
                         ids=["G4-D128-bs16", "G1-D64-bs32-short", "G8-D128-bs32", "G2-D64-bs16",
                              "G1-D64-bs32", "G16-D128-bs16"])
@pytest.mark.parametrize("kind", KINDS)
def test_q8_prefill(case, kind):
    """Chunked causal prefill over int8 pages (the MFMA kernel for these
    shapes; chunks with q_len * G <= 32 take the split-K decode kernels):
    rows reaching position 0, ragged last tiles, several tiles per row."""
    (lengths, q_lens), hq, hkv, d, bs = case
    wl = _case(lengths, hq, hkv, d, bs)
    wl.prefill = list(enumerate(q_lens))
    wl.decode_seqs = []
    pool, ref = _replay(wl, kind)
    qp = prefill_queries(wl)
    out = to_host_f64(pool.prefill(list(range(len(lengths))), q_lens, to_device(qp, "bf16")))
    r0 = 0
    for s, n in wl.prefill:
        keys, values = ref.gather(s)
        exp = oracle.attention(to_f64(qp[r0:r0 + n], "bf16"), keys, values)
        assert_close(out[r0:r0 + n], exp, *BF16_TOL, what=f"seq {s}")
        r0 += n


@pytest.mark.parametrize("kind", KINDS)
def test_q8_prefill_shared_prefix(kind):
    """Three sequences share a 300-token prefix (its blocks refcounted) and
    prefill 200-row chunks of their own tails over 8-bit pages."""
    from paged_kv_cache_block_amd import DevicePool
    hq, hkv, d, bs = 32, 8, 128, 16
    nb = 120
    order = np.random.default_rng(9).permutation(nb).astype(np.int32)
    pool = DevicePool(nb, bs, hkv, d, dtype=kind, allocation_order=order)
    ref = _oracle_pool(nb, bs, hkv, d, order, kind)
    rng = np.random.default_rng(10)
    draw = lambda shape: bf16_round(rng.standard_normal(shape).astype(np.float32))
    def put(s, n):
        k, v = draw((n, hkv, d)), draw((n, hkv, d))
        slots = pool.append(s, n)
        assert slots.tolist() == ref.append(s, n)
        pool.write(slots, to_device(k, "bf16"), to_device(v, "bf16"))
        ref.write(slots, to_f64(k, "bf16"), to_f64(v, "bf16"))
    pool.create(0)
    ref.create(0)
    put(0, 300)
    for s in (1, 2):
        pool.share(0, s, 300)
        ref.share(0, s, 300)
    for s, n in ((0, 200), (1, 211), (2, 200)):
        put(s, n)
    q_lens = [200, 211, 200]
    qp = draw((sum(q_lens), hq, d))
    out = to_host_f64(pool.prefill([0, 1, 2], q_lens, to_device(qp, "bf16")))
    r0 = 0
    for s, n in zip((0, 1, 2), q_lens):
        keys, values = ref.gather(s)
        exp = oracle.attention(to_f64(qp[r0:r0 + n], "bf16"), keys, values)
        assert_close(out[r0:r0 + n], exp, *BF16_TOL, what=f"seq {s}")
        r0 += n


# ------------------------------------------------------------ full size
@pytest.mark.parametrize("kind", KINDS)
def test_q8_full_size_prefix_prefill_sampled_rows(kind):
    """16 x (4096 shared + 512 own) tokens in 8-bit pages, 32/8 heads, d 128,
    bs 16: the 512-row chunks of all sequences in one call; sampled rows
    against the oracle over the dequantised rows."""
    wl = prefix_prefill()
    log(f"q8 prefix_prefill full {kind}: build")
    pool, _ = _replay(wl, kind, mirror=False)
    qp = prefill_queries(wl)
    seqs = [s for s, _ in wl.prefill]
    q_lens = [n for _, n in wl.prefill]
    log("q8 prefix_prefill full: prefill")
    out = to_host_f64(pool.prefill(seqs, q_lens, to_device(qp, "bf16")))
    torch.cuda.synchronize()
    sample_seqs = [0, 9, 15]
    rows = logical_kv(wl, sample_seqs)
    rng = np.random.default_rng(2)
    log("q8 prefix_prefill full: oracle on sampled rows")
    for s in sample_seqs:
        K, V = (_fake_quant(to_f64(x, "bf16"), kind) for x in rows[s])
        L = K.shape[0]
        for t in sorted(set([0, 1, 15, 16, 255, 511] + list(rng.integers(0, 512, 5)))):
            r = s * 512 + t
            vis = L - 512 + t + 1
            exp = oracle.attention(to_f64(qp[r:r + 1], "bf16"), K[:vis], V[:vis])[0]
            assert_close(out[r], exp, *BF16_TOL, what=f"seq {s} row {t}")


@pytest.mark.parametrize("kind", KINDS)
def test_q8_full_size_gqa_decode_step_sampled(kind):
    """32 x U[1, 8192], 32/8 heads, d 128, bs 16 in 8-bit pages, one fused
    decode step as the benchmark times it; sampled sequences against the
    oracle (codes bit-exact, outputs within tolerance)."""
    wl = gqa_decode()
    log(f"q8 full size {kind}: build")
    pool, _ = _replay(wl, kind, mirror=False)
    seqs = list(wl.decode_seqs)
    lengths = wl.final_lengths()
    sample = sorted({int(np.argmax([lengths[s] for s in seqs])), int(np.argmin([lengths[s] for s in seqs])),
                     3, 17, 30})
    rng = np.random.default_rng(77)
    k_new = bf16_round(rng.standard_normal((32, 8, 128)).astype(np.float32))
    v_new = bf16_round(rng.standard_normal((32, 8, 128)).astype(np.float32))
    q = decode_queries(wl, seqs)
    log("q8 full size: decode step")
    out, slots = pool.decode_step(seqs, to_device(k_new, "bf16"), to_device(v_new, "bf16"), to_device(q, "bf16"))
    got = to_host_f64(out)
    kc, ks, vc, vs = _device_codes(pool)
    rows = logical_kv(wl, sample)
    bs = wl.block_size
    for s in sample:
        K = np.concatenate([to_f64(rows[s][0], "bf16"), to_f64(k_new[s:s + 1], "bf16")])
        V = np.concatenate([to_f64(rows[s][1], "bf16"), to_f64(v_new[s:s + 1], "bf16")])
        table = pool.block_table(s)
        n = K.shape[0]
        blk = table[np.arange(n) // bs]
        off = np.arange(n) % bs
        codes, scale = _quant(K, kind)
        np.testing.assert_array_equal(kc[blk, off], codes, err_msg=f"K codes seq {s}")
        np.testing.assert_array_equal(ks[blk, off], oracle.stored_scale(scale[..., 0]).astype(np.float32))
        codes, scale = _quant(V, kind)
        np.testing.assert_array_equal(vc[blk, off], codes, err_msg=f"V codes seq {s}")
        want = oracle.attention(to_f64(q[s:s + 1], "bf16"), _fake_quant(K, kind), _fake_quant(V, kind))[0]
        assert_close(got[s], want, *BF16_TOL, what=f"seq {s} (L={n})")
