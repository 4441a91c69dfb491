"""GPU parity of decode over sequences built through the prefix cache: the
attached (shared) blocks hold the K/V rows the first request stored, the
rest are the new request's own rows.

Source: vladkulikov.com notebook "Модуль 10", prefix-caching cell (keys over
all preceding tokens at complete block boundaries).  Bar: tables and
refcounts bit-exact against the oracle; outputs within (2e-3, 1e-2).
"""

import numpy as np
import pytest

import oracle
from oracle import PrefixCache
from synth.workloads import bf16_round, to_f64

from gpu_support import BF16_TOL, assert_close, to_device, to_host_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_block_amd import abi
    abi.load()


@pytest.mark.parametrize("kv", ["bf16", "i8", "fp8"])
def test_decode_after_prefix_attach(kv):
    from paged_kv_cache_block_amd import DevicePool
    hq, hkv, d, bs, nb = 32, 8, 128, 16, 64
    order = np.random.default_rng(8).permutation(nb).astype(np.int32)
    pool = DevicePool(nb, bs, hkv, d, dtype=kv, allocation_order=order)
    ref = oracle.Pool(nb, bs, hkv, d, allocation_order=order, quant_bits=8 if kv in ("i8", "fp8") else None,
                     quant_fp8=kv == "fp8")
    cache = PrefixCache(ref)
    rng = np.random.default_rng(9)
    prompt = [int(x) for x in rng.integers(0, 50, size=70)]
    requests = [prompt, prompt[:40] + [7] * 25, prompt + [3] * 9, [1] + prompt]
    hits = []
    for i, tokens in enumerate(requests):
        hit = pool.prefix_attach(i, tokens, "tenant", "model-r1")
        assert hit == cache.attach(i, tokens, "tenant", "model-r1")
        hits.append(hit)
        n = len(tokens) - hit
        k = bf16_round(rng.standard_normal((n, hkv, d)).astype(np.float32))
        v = bf16_round(rng.standard_normal((n, hkv, d)).astype(np.float32))
        slots = pool.append(i, n)
        assert slots.tolist() == ref.append(i, n)
        pool.write(slots, to_device(k, "bf16"), to_device(v, "bf16"))
        ref.write(slots, to_f64(k, "bf16"), to_f64(v, "bf16"))
        assert pool.prefix_register(i, tokens, "tenant", "model-r1") == cache.register(i, tokens, "tenant", "model-r1")
    assert hits == [0, 32, 64, 0]
    assert [pool.prefix_lookup(t, "tenant", "model-r1") for t in requests] == [64] * 4
    for i in range(4):
        assert pool.block_table(i).tolist() == ref.tables[i]
    assert [pool.refcount(b) for b in range(nb)] == ref.refs.tolist()
    q = bf16_round(rng.standard_normal((4, hq, d)).astype(np.float32))
    got = to_host_f64(pool.decode([0, 1, 2, 3], to_device(q, "bf16")))
    for i in range(4):
        want = oracle.paged_attention(ref, i, to_f64(q[i:i + 1], "bf16"))[0]
        assert_close(got[i], want, *BF16_TOL, what=f"request {i}")
    pool.validate()
