"""Paged attention over a refcounted KV block pool, native to AMD MI355X.

The product is ``libpagedattn.so`` (C ABI in ``include/pagedattn.h``):
host bookkeeping of the pool in C++ and hand-written gfx950 HIP kernels for
the cache writes, decode (split-K over pages with a log-sum-exp merge) and
chunked causal prefill.  This package holds its sources (``csrc/``), the build
step (``build.py``), the ctypes binding (``abi``) and a torch-backed
convenience pool (``DevicePool``).  Loading fails loudly if the library has
not been built; there is no CPU fallback.
"""

from . import abi
from .abi import (PagedAttnError, UnknownSequenceError, SequenceExistsError, InvalidArgumentError,
                  OutOfBlocksError, DeviceError)
from .pool import DevicePool

__all__ = [
    "abi",
    "DevicePool",
    "PagedAttnError",
    "UnknownSequenceError",
    "SequenceExistsError",
    "InvalidArgumentError",
    "OutOfBlocksError",
    "DeviceError",
]
