"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This package holds no arithmetic of the method itself: it draws random
numbers, rounds them to the input dtype, and lists the pool operations of
each workload (create / append / share) and the attention calls to make.  The
pool model, slot mapping and attention live in ``oracle`` (reference) and in
the HIP library (product); neither is imported here.
"""

from .workloads import (
    Workload,
    bf16_round,
    bf16_bits_to_f32,
    tiny_fp32,
    gqa_decode,
    long_decode,
    prefix_prefill,
    heavy_tail,
    WORKLOADS,
    append_stream,
    decode_queries,
    prefill_queries,
    logical_kv,
    prefix_trace_requests,
)

__all__ = [
    "Workload",
    "bf16_round",
    "bf16_bits_to_f32",
    "tiny_fp32",
    "gqa_decode",
    "long_decode",
    "prefix_prefill",
    "heavy_tail",
    "WORKLOADS",
    "append_stream",
    "decode_queries",
    "prefill_queries",
    "logical_kv",
    "prefix_trace_requests",
]
