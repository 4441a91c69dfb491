"""GPU parity of prefill run chunk by chunk: each chunk appends its rows
(pa_append), stores their K/V (pa_reshape_and_cache) and runs pa_prefill_chunk
for them, and the chunks' outputs together must equal one causal prefill
of all the rows over the final cache.

Source: the vladkulikov.com notebook "Модуль 10", prefix-and-interference
cell (the chunks of a prefill hold exactly the causal query-key pairs of one
prefill), and docs.rs ferrum-kv 0.4.0 src/attention.rs, paged_attention with
q_tokens > 1 (row t sees keys j <= kv_len - q_tokens + t).  The chunk sizes
mix the MFMA prefill kernel (128, 200 and 176 rows) with the split-K decode
kernels (an 8-row chunk: 8 rows x 4 heads = 32 MFMA columns), so successive
plans and workspaces of both paths meet on one pool.  Bar: slots and tables
bit-exact against the oracle pool; every output row x head within (2e-3,
1e-2) of the float64 oracle's one-shot attention.
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


CHUNKS = [128, 200, 8, 176]  # 512 rows per sequence


@pytest.mark.parametrize("kv", ["bf16", "i8", "fp8"])
def test_chunk_by_chunk_prefill_equals_one_shot(kv):
    from paged_kv_cache_block_amd import DevicePool
    hq, hkv, d, bs = 32, 8, 128, 16
    prefixes = [1000, 517]          # cached tokens before the chunks
    total = sum(CHUNKS)
    nb = sum(-(-(p + total) // bs) for p in prefixes) + 8
    order = np.random.default_rng(31).permutation(nb).astype(np.int32)
    pool = DevicePool(nb, bs, hkv, d, dtype=kv, allocation_order=order)
    ref = oracle.Pool(nb, bs, hkv, d, allocation_order=order, quant_bits=8 if kv in ("i8", "fp8") else None,
                      quant_fp8=kv == "fp8")
    rng = np.random.default_rng(32)
    seqs = list(range(len(prefixes)))

    def store(s, n):
        k = bf16_round(rng.standard_normal((n, hkv, d)).astype(np.float32))
        v = bf16_round(rng.standard_normal((n, hkv, d)).astype(np.float32))
        slots = pool.append(s, n)
        want = ref.append(s, n)
        assert slots.tolist() == want
        pool.write(slots, to_device(k, "bf16"), to_device(v, "bf16"))
        ref.write(want, to_f64(k, "bf16"), to_f64(v, "bf16"))

    for s, p in enumerate(prefixes):
        pool.create(s)
        ref.create(s)
        store(s, p)
    q_all = {s: bf16_round(rng.standard_normal((total, hq, d)).astype(np.float32)) for s in seqs}
    got = {s: [] for s in seqs}
    r0 = 0
    for n in CHUNKS:
        log(f"{kv}: chunk of {n} rows per sequence at row {r0}")
        for s in seqs:
            store(s, n)
        q = np.concatenate([q_all[s][r0:r0 + n] for s in seqs])
        out = pool.prefill(seqs, [n] * len(seqs), to_device(q, "bf16"))
        host = to_host_f64(out)
        for i, s in enumerate(seqs):
            got[s].append(host[i * n:(i + 1) * n])
        r0 += n
    torch.cuda.synchronize()
    for s in seqs:
        assert pool.block_table(s).tolist() == ref.tables[s]
        keys, values = ref.gather(s)
        want = oracle.attention(to_f64(q_all[s], "bf16"), keys, values)   # one prefill of all 512 rows
        assert_close(np.concatenate(got[s]), want, *BF16_TOL, what=f"{kv} seq {s}")
    pool.validate()
    pool.close()
