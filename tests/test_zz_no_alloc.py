"""GPU test of pa_decode_step_noalloc, the decode step whose workspace is
the library's static per-GPU scratch array (for callers that cannot
allocate memory).

Two pools are built identically; each step runs pa_decode_step (caller
workspace) on one and pa_decode_step_noalloc on the other with the same
inputs.  Slots, tables and refcounts must be equal, outputs bit-identical
(the same kernels over the same plan), and both within (2e-3, 1e-2) of the
float64 oracle ([ferrum] paged_attention, q_tokens = 1).  Two calls in a
row, the second with a smaller batch; then a batch whose workspace exceeds
the scratch is rejected with the pools unchanged.
"""

import numpy as np
import pytest

import oracle
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


def _pair(lengths, hq, hkv, d, bs, kv, seed):
    """Two identical device pools (and the oracle's) holding the same rows;
    the last sequence is a fork of sequence 1, so the first step copies a
    shared partial tail."""
    from paged_kv_cache_block_amd import DevicePool
    nb = int(sum(-(-n // bs) for n in lengths) * 2 + 64)
    order = np.random.default_rng(seed).permutation(nb).astype(np.int32)
    pools = [DevicePool(nb, bs, hkv, d, dtype=kv, allocation_order=order) for _ in range(2)]
    ref = oracle.Pool(nb, bs, hkv, d, allocation_order=order, quant_bits=8 if kv in ("i8", "fp8") else None,
                      quant_fp8=kv == "fp8")
    rng = np.random.default_rng(seed + 1)
    for s, n in enumerate(lengths):
        k = bf16_round(rng.standard_normal((n, hkv, d)).astype(np.float32))
        v = bf16_round(rng.standard_normal((n, hkv, d)).astype(np.float32))
        ref.create(s)
        want = ref.append(s, n)
        ref.write(want, to_f64(k, "bf16"), to_f64(v, "bf16"))
        for p in pools:
            p.create(s)
            slots = p.append(s, n)
            assert slots.tolist() == want
            p.write(slots, to_device(k, "bf16"), to_device(v, "bf16"))
    fork = len(lengths)
    ref.fork(1, fork)
    for p in pools:
        p.fork(1, fork)
    torch.cuda.synchronize()
    return pools, ref, rng, list(range(len(lengths))) + [fork]


def _step_both(pools, ref, rng, seqs, hq, hkv, d, what):
    B = len(seqs)
    k = bf16_round(rng.standard_normal((B, hkv, d)).astype(np.float32))
    v = bf16_round(rng.standard_normal((B, hkv, d)).astype(np.float32))
    q = bf16_round(rng.standard_normal((B, hq, d)).astype(np.float32))
    kd, vd, qd = to_device(k, "bf16"), to_device(v, "bf16"), to_device(q, "bf16")
    out_ws = torch.full_like(qd, float("nan"))
    out_na = torch.full_like(qd, float("nan"))
    log(f"{what}: pa_decode_step on pool 0, B {B}")
    _, slots_ws = pools[0].decode_step(seqs, kd, vd, qd, out_ws)
    log(f"{what}: pa_decode_step_noalloc on pool 1, B {B}")
    _, slots_na = pools[1].decode_step_noalloc(seqs, kd, vd, qd, out_na)
    torch.cuda.synchronize()
    want_slots = [slot for s in seqs for slot in ref.append(s, 1)]
    assert slots_ws.tolist() == want_slots
    assert slots_na.tolist() == want_slots
    ref.write(want_slots, to_f64(k, "bf16"), to_f64(v, "bf16"))
    for s in seqs:
        assert pools[0].block_table(s).tolist() == pools[1].block_table(s).tolist() == ref.tables[s]
    for blk in range(ref.num_blocks):
        assert pools[0].refcount(blk) == pools[1].refcount(blk) == ref.refs[blk]
    assert torch.equal(out_ws.view(torch.int16), out_na.view(torch.int16)), f"{what}: outputs differ"
    got = to_host_f64(out_na)
    for i, s in enumerate(seqs):
        keys, values = ref.gather(s)
        want = oracle.attention(to_f64(q[i:i + 1], "bf16"), keys, values)[0]
        assert_close(got[i], want, *BF16_TOL, what=f"{what} row {i}")
    for p in pools:
        p.validate()


CASES = [
    # lengths, Hq, Hkv, D, bs, pages
    ([1, 15, 700, 3000, 9000], 32, 8, 128, 16, "bf16"),
    ([5, 40, 2049, 777], 16, 16, 64, 32, "bf16"),
    ([3, 77, 3000, 130], 32, 8, 128, 16, "i8"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[5]}-hq{c[1]}-d{c[3]}-bs{c[4]}")
def test_noalloc_step_matches_decode_step(case):
    lengths, hq, hkv, d, bs, kv = case
    pools, ref, rng, seqs = _pair(lengths, hq, hkv, d, bs, kv, seed=41)
    _step_both(pools, ref, rng, seqs, hq, hkv, d, "call 1 (whole batch, copy-on-write of the fork)")
    _step_both(pools, ref, rng, seqs[1:4], hq, hkv, d, "call 2 (smaller batch)")
    for p in pools:
        p.close()


def _pool_above_the_scratch():
    """A pool and batch whose decode step needs more workspace than the
    static scratch: 32 query heads over 1 KV head (the split-K partial rows
    hold 32 x 130 floats per page range), with the batch grown until the
    page ranges the plan picks add up to more than 16 MiB of partials."""
    from paged_kv_cache_block_amd import DevicePool, abi
    hq = 32
    for B, L in ((16, 16384), (127, 16383), (255, 16383)):
        pool = DevicePool(B * (L // 16 + 2) + 16, 16, 1, 128, dtype="bf16")
        seqs = list(range(B))
        for s in seqs:
            pool.create(s)
            pool.append(s, L)
        need = abi.pa_decode_step_workspace_bytes(pool.handle, seqs, hq)
        if need > abi.PA_NOALLOC_SCRATCH_BYTES:
            return pool, seqs, hq, need
        pool.close()
    pytest.fail("no batch of the list needs more workspace than the static scratch")


def test_noalloc_step_rejects_workspace_above_the_scratch():
    """A step whose workspace exceeds the static scratch fails before
    anything changes (no rows are written, so none are needed)."""
    from paged_kv_cache_block_amd.abi import InvalidArgumentError
    pool, seqs, hq, need = _pool_above_the_scratch()
    B = len(seqs)
    before = [pool.seq_len(s) for s in seqs]
    stats = pool.stats()
    new = torch.zeros((B, 1, 128), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((B, hq, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    log(f"noalloc rejection: {B} sequences, workspace {need} bytes above the static scratch")
    with pytest.raises(InvalidArgumentError, match="static scratch"):
        pool.decode_step_noalloc(seqs, new, new, q, out)
    assert [pool.seq_len(s) for s in seqs] == before
    assert pool.stats() == stats
    pool.validate()
    pool.close()
