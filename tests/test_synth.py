"""The seeded input generators: bf16 rounding and the workload recipes."""

import math

import numpy as np
import torch

from synth import (bf16_bits_to_f32, bf16_round, gqa_decode, heavy_tail, logical_kv,
                   long_decode, prefix_prefill, tiny_fp32, append_stream, decode_queries,
                   prefill_queries)


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8, 0.0, -0.0, 3e38], np.float32)])
    ours = bf16_round(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == theirs).all()
    back = bf16_bits_to_f32(ours)
    assert (back == torch.from_numpy(x).to(torch.bfloat16).float().numpy()).all()


def test_recipe_sizes():
    wl = tiny_fp32()
    assert wl.allocation_order.tolist() == [2, 4, 3, 6, 5, 0, 1, 7]
    lengths = np.array(list(gqa_decode().final_lengths().values()))
    assert (lengths.sum(), lengths.min(), lengths.max()) == (130736, 226, 7787)
    assert sum(-(-lengths // 16)) == 8183
    ht = heavy_tail()
    lengths = np.array(list(ht.final_lengths().values()))
    assert (lengths.sum(), lengths.min(), lengths.max()) == (1371446, 17, 32373)
    assert ht.num_blocks == 47758 and sum(-(-lengths // 32)) == 42982
    assert long_decode().final_lengths() == {i: 131072 for i in range(4)}
    pp = prefix_prefill()
    assert pp.final_lengths() == {i: 4608 for i in range(16)}


def test_streams_are_per_sequence_and_deterministic():
    wl = gqa_decode(batch=4, max_len=40, num_blocks=64)
    a = [op for op in append_stream(wl) if op[0] == "append"]
    b = [op for op in append_stream(wl, only={2}) if op[0] == "append"]
    assert b[0][3] is None and (a[2][3] == b[2][3]).all() and (a[2][4] == b[2][4]).all()
    q1 = decode_queries(wl)
    q2 = decode_queries(wl, seqs=[2])
    assert (q1[2] == q2[0]).all()


def test_logical_rows_of_shared_prefix():
    wl = prefix_prefill(batch=3, prefix=10, chunk=3, num_blocks=32, num_heads=2, num_kv_heads=1,
                        head_dim=4, block_size=4)
    rows = logical_kv(wl, [0, 2])
    assert rows[0][0].shape == (13, 1, 4) and rows[2][0].shape == (13, 1, 4)
    assert (rows[0][0][:10] == rows[2][0][:10]).all()
    assert not (rows[0][0][10:] == rows[2][0][10:]).all()
    q = prefill_queries(wl)
    assert q.shape == (9, 2, 4)


def test_outlier_rows_scaled_by_eight():
    wl = heavy_tail(batch=4, max_len=2000)
    ops = [op for op in append_stream(wl) if op[0] == "append"]
    k = bf16_bits_to_f32(np.concatenate([op[3] for op in ops]))
    norms = np.abs(k).max(axis=2)
    frac = (norms > 6).mean()
    assert 0.003 < frac < 0.03
