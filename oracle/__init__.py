"""Float64 CPU oracle for paged attention over a refcounted KV block pool.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain reference the HIP
path is checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with
``paged_kv_cache_block_amd`` (no kernels, headers, helpers, tables or
pre/post-processing) and never imports it; the product path never imports
this package.

Sources (the pages, cited by title and section):

* abhik.ai, "examples/pagedattention.py" -- the ``KVPool`` regions
  physical_pool, logical_address, append_or_allocate, fork_prefix,
  copy_on_write, paged_attention, release_sequence (single-head float64
  ownership mechanics).
* vladkulikov.com course notebook "Модуль 10. KV-кэши и эффективный инференс"
  -- ``PagedKVPool`` (preflighted multi-token append, share_prefix, release,
  fill accounting, ``validate``) and its embedded reference contract; its
  KV-compression experiment (per-row absmax codes, ``fake_quantize_rows``);
  its prefix-caching cell (block keys, ``run_prefix_trace``); its
  eviction cell (the streaming keep rule) and explicit window caches.
* docs.rs ferrum-kv 0.4.0 ``src/attention.rs`` -- ``paged_attention``
  (GQA head grouping, 1/sqrt(head_dim) scale, bottom-right causal mask).
* CMU 11-667 lecture 19 ``infer_world.py``, section 3 "online softmax and
  tiled attention" -- ``online_softmax_stats`` / ``tiled_attention`` /
  ``reference_attention``.

Modules:

* :mod:`oracle.pool` -- the pool model (integer bookkeeping, exact) with its
  own float64 K/V storage.
* :mod:`oracle.quant` -- per-row absmax quantisation of K/V rows (codes,
  fp32 scales, read-back values); a ``Pool(quant_bits=8)`` stores through it.
* :mod:`oracle.fp8` -- the same row scheme with 8-bit float codes (E4M3,
  no infinities; a reading beyond the pages, pinned to the format's
  definition); a ``Pool(quant_fp8=True)`` stores through it.
* :mod:`oracle.prefix` -- prefix-hash block reuse: complete-block keys
  (scope, revision, all preceding tokens) mapped to pinned pool blocks.
* :mod:`oracle.window` -- sliding-window attention with sinks (the keep
  rule as ``window_keep``) over the resident rows of a windowed pool
  sequence.
* :mod:`oracle.attention` -- the attention definition, its online-softmax
  restatement, the log-sum-exp merge of partial results and a pure-Python
  brute force for tiny inputs.

Parity status: every function here is pinned by ``-m "not gpu"`` tests
(printed trace values, closed forms, brute force, invariants).  No function is
"parity unpinned".
"""

from .pool import Pool, OutOfBlocks, UnknownSequence, SequenceExists
from .quant import (
    code_limit,
    quantize_rows,
    stored_scale,
    dequantize_rows,
    fake_quantize_rows,
    packed_bytes,
)
from .fp8 import (
    E4M3_MAX,
    e4m3_decode,
    e4m3_round,
    e4m3_encode,
    quantize_rows_fp8,
    dequantize_rows_fp8,
    fake_quantize_rows_fp8,
)
from .prefix import BlockKey, PrefixCache, block_key, run_prefix_trace
from .window import window_keep, windowed_attention
from .attention import (
    attention,
    paged_attention,
    combine_stats,
    online_softmax_stats,
    tiled_attention,
    brute_force_attention,
    partial_attention,
    merge_partials,
)

__all__ = [
    "Pool",
    "OutOfBlocks",
    "UnknownSequence",
    "SequenceExists",
    "attention",
    "paged_attention",
    "combine_stats",
    "online_softmax_stats",
    "tiled_attention",
    "brute_force_attention",
    "partial_attention",
    "merge_partials",
    "code_limit",
    "quantize_rows",
    "stored_scale",
    "dequantize_rows",
    "fake_quantize_rows",
    "packed_bytes",
    "E4M3_MAX",
    "e4m3_decode",
    "e4m3_round",
    "e4m3_encode",
    "quantize_rows_fp8",
    "dequantize_rows_fp8",
    "fake_quantize_rows_fp8",
    "PrefixCache",
    "BlockKey",
    "block_key",
    "run_prefix_trace",
    "window_keep",
    "windowed_attention",
]
