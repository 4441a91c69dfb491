"""ctypes binding of libpagedattn.so, one Python function per C entry point.

Argument marshalling only: host arrays become numpy buffers, device buffers
are passed by address (an int, or any object with ``data_ptr()`` such as a
torch tensor), streams by handle (an int, ``None`` for the default stream,
or a torch stream).  Every computation happens in the library.  A failing
call raises :class:`PagedAttnError` (a subclass matching the status: an
unknown id is also a ``KeyError``, an existing id or a bad argument a
``ValueError``, pool exhaustion a ``MemoryError``, a HIP failure a
``RuntimeError``).  Loading fails loudly when the library is not built.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedattn.so")

PA_OK = 0
PA_ERR_INVALID_ARG = -1
PA_ERR_UNKNOWN_SEQ = -2
PA_ERR_SEQ_EXISTS = -3
PA_ERR_OUT_OF_BLOCKS = -4
PA_ERR_DEVICE = -5

PA_DTYPE_F32 = 0
PA_DTYPE_BF16 = 1
PA_DTYPE_I8 = 2
PA_DTYPE_FP8 = 3

PA_KERNEL_DECODE = 0
PA_KERNEL_MERGE = 1
PA_KERNEL_PREFILL = 2
PA_KERNEL_CACHE = 3
PA_KERNEL_COPY = 4
PA_KERNEL_COUNT = 5


class PagedAttnError(Exception):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


class UnknownSequenceError(PagedAttnError, KeyError):
    pass


class SequenceExistsError(PagedAttnError, ValueError):
    pass


class InvalidArgumentError(PagedAttnError, ValueError):
    pass


class OutOfBlocksError(PagedAttnError, MemoryError):
    pass


class DeviceError(PagedAttnError, RuntimeError):
    pass


_ERRORS = {
    PA_ERR_INVALID_ARG: InvalidArgumentError,
    PA_ERR_UNKNOWN_SEQ: UnknownSequenceError,
    PA_ERR_SEQ_EXISTS: SequenceExistsError,
    PA_ERR_OUT_OF_BLOCKS: OutOfBlocksError,
    PA_ERR_DEVICE: DeviceError,
}


class pa_pool_desc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class pa_pool_stats(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int64) for name in (
        "allocated_blocks", "free_blocks", "physical_capacity_tokens", "physical_payload_tokens",
        "logical_tokens", "internal_waste_tokens", "sharing_savings_tokens")]


_c_void_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_size = ctypes.c_size_t
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)

# name: (restype, argtypes)
SIGNATURES = {
    "pa_pool_bytes": (_size, [ctypes.POINTER(pa_pool_desc)]),
    "pa_pool_create": (_i32, [ctypes.POINTER(pa_pool_desc), _c_void_p, _c_void_p, _c_void_p, ctypes.POINTER(_c_void_p)]),
    "pa_pool_destroy": (None, [_c_void_p]),
    "pa_pool_reserve_staging": (_i32, [_c_void_p, _size, ctypes.POINTER(_size)]),
    "pa_seq_create": (_i32, [_c_void_p, _i64]),
    "pa_append": (_i32, [_c_void_p, _i64, _i32, _c_void_p]),
    "pa_append_batch": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i32, _c_void_p]),
    "pa_share": (_i32, [_c_void_p, _i64, _i64, _i32]),
    "pa_fork": (_i32, [_c_void_p, _i64, _i64]),
    "pa_release": (_i32, [_c_void_p, _i64]),
    "pa_seq_set_window": (_i32, [_c_void_p, _i64, _i32, _i32]),
    "pa_truncate": (_i32, [_c_void_p, _i64, _i32]),
    "pa_prefix_lookup": (_i32, [_c_void_p, ctypes.c_char_p, ctypes.c_char_p, _c_void_p, _i32, _i32p]),
    "pa_prefix_attach": (_i32, [_c_void_p, _i64, ctypes.c_char_p, ctypes.c_char_p, _c_void_p, _i32, _i32p]),
    "pa_prefix_register": (_i32, [_c_void_p, _i64, ctypes.c_char_p, ctypes.c_char_p, _c_void_p, _i32, _i32p]),
    "pa_prefix_clear": (_i32, [_c_void_p, _i32p]),
    "pa_prefix_entries": (_i32, [_c_void_p, _i64p]),
    "pa_pending_copies": (_i32, [_c_void_p, _c_void_p, _i32, _i32p]),
    "pa_flush_copies": (_i32, [_c_void_p, _c_void_p]),
    "pa_reshape_and_cache": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _c_void_p]),
    "pa_pool_set_slot_checks": (_i32, [_c_void_p, ctypes.c_int, _c_void_p]),
    "pa_decode_workspace_bytes": (_size, [_c_void_p, _c_void_p, _i32, _i32]),
    "pa_decode": (_i32, [_c_void_p, _c_void_p, _i32, _i32, _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p]),
    "pa_decode_step_workspace_bytes": (_size, [_c_void_p, _c_void_p, _i32, _i32]),
    "pa_decode_step": (_i32, [_c_void_p, _c_void_p, _i32, _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p, _c_void_p]),
    "pa_decode_step_noalloc": (_i32, [_c_void_p, _c_void_p, _i32, _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "pa_verify_step_workspace_bytes": (_size, [_c_void_p, _c_void_p, _c_void_p, _i32, _i32]),
    "pa_verify_step": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i32, _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p, _c_void_p]),
    "pa_prefill_workspace_bytes": (_size, [_c_void_p, _c_void_p, _c_void_p, _i32, _i32]),
    "pa_prefill_chunk": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i32, _i32, _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p]),
    "pa_seq_len": (_i32, [_c_void_p, _i64, _i32p]),
    "pa_block_table": (_i32, [_c_void_p, _i64, _c_void_p, _i32, _i32p]),
    "pa_refcount": (_i32, [_c_void_p, _i32, _i32p]),
    "pa_stats": (_i32, [_c_void_p, ctypes.POINTER(pa_pool_stats)]),
    "pa_validate": (_i32, [_c_void_p]),
    "pa_sequences": (_i32, [_c_void_p, _c_void_p, _i32, _i32p]),
    "pa_decode_work_items": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32p, _c_void_p, _i32, _i32p,
                                    _c_void_p, _i64, _i64p]),
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_timing_enable": (_i32, [ctypes.c_int]),
    "pa_timing_reset": (_i32, []),
    "pa_timing_select": (_i32, [ctypes.c_uint32]),
    "pa_timing_read": (_i32, [_i32, ctypes.POINTER(ctypes.c_double), _i64p]),
    "pa_timing_samples": (_i32, [_i32, ctypes.POINTER(ctypes.c_float), _i64, _i64p]),
}

_lib = None


def load():
    """Load libpagedattn.so (once).  Raises ImportError if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built: run `python -m paged_kv_cache_block_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status):
    if status != PA_OK:
        msg = load().pa_last_error().decode("utf-8", "replace")
        raise _ERRORS.get(status, PagedAttnError)(status, msg)


def _addr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if hasattr(x, "cuda_stream"):
        return x.cuda_stream
    raise TypeError(f"cannot take a device address of {type(x).__name__}")


def _stream(s):
    if s is None:
        return None
    if hasattr(s, "cuda_stream"):
        return s.cuda_stream
    return int(s)


def _ptr(arr):
    """Address of a contiguous numpy array's data, passed as a void pointer
    (cheaper than building a typed ctypes pointer on every call)."""
    return arr.__array_interface__["data"][0]


def _i64_array(values):
    arr = values
    if not (isinstance(arr, np.ndarray) and arr.dtype == np.int64 and arr.flags.c_contiguous):
        arr = np.ascontiguousarray(np.asarray(values, dtype=np.int64))
    return arr, _ptr(arr)


def _i32_array(values):
    arr = values
    if not (isinstance(arr, np.ndarray) and arr.dtype == np.int32 and arr.flags.c_contiguous):
        arr = np.ascontiguousarray(np.asarray(values, dtype=np.int32))
    return arr, _ptr(arr)


# --------------------------------------------------------------------- pool
def make_desc(num_blocks, block_size, num_kv_heads, head_dim, dtype):
    return pa_pool_desc(num_blocks, block_size, num_kv_heads, head_dim, dtype)


def pa_pool_bytes(desc):
    return int(load().pa_pool_bytes(ctypes.byref(desc)))


def pa_pool_create(desc, allocation_order=None, k_pool=None, v_pool=None):
    out = _c_void_p()
    order_ptr = None
    if allocation_order is not None:
        order, order_ptr = _i32_array(allocation_order)
    _check(load().pa_pool_create(ctypes.byref(desc), order_ptr, _addr(k_pool), _addr(v_pool),
                                 ctypes.byref(out)))
    return out.value


def pa_pool_destroy(pool):
    load().pa_pool_destroy(pool)


def pa_pool_reserve_staging(pool, plan_bytes):
    """Grow the pool's pinned staging buffers to ``plan_bytes``; returns the size reserved."""
    reserved = _size()
    _check(load().pa_pool_reserve_staging(pool, plan_bytes, ctypes.byref(reserved)))
    return reserved.value


def pa_seq_create(pool, seq):
    _check(load().pa_seq_create(pool, seq))


def pa_append(pool, seq, n_tokens):
    slots = np.empty(max(n_tokens, 0), dtype=np.int64)
    _check(load().pa_append(pool, seq, n_tokens, _ptr(slots) if n_tokens > 0 else None))
    return slots


def pa_append_batch(pool, seqs, n_tokens, slots_out=None):
    """Batched append; ``slots_out`` (int64, contiguous) may be passed to reuse a buffer."""
    arr, ptr = _i64_array(seqs)
    ns, nptr = _i32_array(n_tokens)
    total = int(ns.sum()) if len(ns) else 0
    if slots_out is None:
        slots_out = np.empty(total, dtype=np.int64)
    assert slots_out.dtype == np.int64 and slots_out.flags.c_contiguous and slots_out.size >= total
    _check(load().pa_append_batch(pool, ptr, nptr, len(arr),
                                  _ptr(slots_out) if total else None))
    return slots_out[:total]


def pa_share(pool, src, dst, prefix_tokens):
    _check(load().pa_share(pool, src, dst, prefix_tokens))


def pa_fork(pool, src, dst):
    _check(load().pa_fork(pool, src, dst))


def pa_release(pool, seq):
    _check(load().pa_release(pool, seq))


def pa_seq_set_window(pool, seq, sink_tokens, recent_tokens):
    _check(load().pa_seq_set_window(pool, seq, sink_tokens, recent_tokens))


def pa_truncate(pool, seq, new_length):
    _check(load().pa_truncate(pool, seq, new_length))


def _bytes(x):
    return x if isinstance(x, bytes) else str(x).encode()


def pa_prefix_lookup(pool, scope, revision, tokens):
    """Hit (tokens) of ``tokens`` in the pool's prefix cache."""
    arr, ptr = _i32_array(tokens)
    hit = _i32()
    _check(load().pa_prefix_lookup(pool, _bytes(scope), _bytes(revision), ptr, len(arr), ctypes.byref(hit)))
    return hit.value


def pa_prefix_attach(pool, seq, scope, revision, tokens):
    """New sequence holding the cached blocks of its hit; returns the hit."""
    arr, ptr = _i32_array(tokens)
    hit = _i32()
    _check(load().pa_prefix_attach(pool, seq, _bytes(scope), _bytes(revision), ptr, len(arr),
                                   ctypes.byref(hit)))
    return hit.value


def pa_prefix_register(pool, seq, scope, revision, tokens):
    """Cache the complete blocks of ``seq``'s first len(tokens) positions;
    returns the number of new keys."""
    arr, ptr = _i32_array(tokens)
    added = _i32()
    _check(load().pa_prefix_register(pool, seq, _bytes(scope), _bytes(revision), ptr, len(arr),
                                     ctypes.byref(added)))
    return added.value


def pa_prefix_clear(pool):
    n = _i32()
    _check(load().pa_prefix_clear(pool, ctypes.byref(n)))
    return n.value


def pa_prefix_entries(pool):
    n = _i64()
    _check(load().pa_prefix_entries(pool, ctypes.byref(n)))
    return n.value


def pa_pending_copies(pool):
    n = _i32()
    _check(load().pa_pending_copies(pool, None, 0, ctypes.byref(n)))
    pairs = np.empty((n.value, 2), dtype=np.int32)
    if n.value:
        _check(load().pa_pending_copies(pool, _ptr(pairs), n.value, ctypes.byref(n)))
    return [tuple(map(int, p)) for p in pairs]


def pa_flush_copies(pool, stream=None):
    _check(load().pa_flush_copies(pool, _stream(stream)))


def pa_reshape_and_cache(pool, k_new, v_new, slots, n, stream=None):
    _check(load().pa_reshape_and_cache(pool, _addr(k_new), _addr(v_new), _addr(slots), n,
                                       _stream(stream)))


def pa_pool_set_slot_checks(pool, on, stream=None):
    _check(load().pa_pool_set_slot_checks(pool, 1 if on else 0, _stream(stream)))


# ---------------------------------------------------------------- attention
def pa_decode_workspace_bytes(pool, seqs, num_heads):
    arr, ptr = _i64_array(seqs)
    return int(load().pa_decode_workspace_bytes(pool, ptr, len(arr), num_heads))


def pa_decode(pool, seqs, num_heads, q, out, ws, ws_bytes, stream=None):
    arr, ptr = _i64_array(seqs)
    _check(load().pa_decode(pool, ptr, len(arr), num_heads, _addr(q), _addr(out), _addr(ws),
                            ws_bytes, _stream(stream)))


def pa_decode_step_workspace_bytes(pool, seqs, num_heads):
    arr, ptr = _i64_array(seqs)
    return int(load().pa_decode_step_workspace_bytes(pool, ptr, len(arr), num_heads))


def pa_decode_step(pool, seqs, num_heads, k_new, v_new, q, out, ws, ws_bytes, stream=None,
                   slots_out=None):
    """Fused decode step; returns the new slots (int64 [B]) when ``slots_out`` is given or True."""
    arr, ptr = _i64_array(seqs)
    sp = None
    if slots_out is True:
        slots_out = np.empty(len(arr), dtype=np.int64)
    if slots_out is not None:
        assert slots_out.dtype == np.int64 and slots_out.size >= len(arr)
        sp = _ptr(slots_out)
    _check(load().pa_decode_step(pool, ptr, len(arr), num_heads, _addr(k_new), _addr(v_new), _addr(q),
                                 _addr(out), _addr(ws), ws_bytes, sp, _stream(stream)))
    return slots_out


def pa_decode_step_noalloc(pool, seqs, num_heads, k_new, v_new, q, out, stream=None, slots_out=None):
    """pa_decode_step with the library's static scratch as its workspace;
    returns the new slots when ``slots_out`` is given or True."""
    arr, ptr = _i64_array(seqs)
    sp = None
    if slots_out is True:
        slots_out = np.empty(len(arr), dtype=np.int64)
    if slots_out is not None:
        assert slots_out.dtype == np.int64 and slots_out.size >= len(arr)
        sp = _ptr(slots_out)
    _check(load().pa_decode_step_noalloc(pool, ptr, len(arr), num_heads, _addr(k_new), _addr(v_new),
                                         _addr(q), _addr(out), sp, _stream(stream)))
    return slots_out


PA_NOALLOC_SCRATCH_BYTES = 16 << 20


def pa_verify_step_workspace_bytes(pool, seqs, q_lens, num_heads):
    arr, ptr = _i64_array(seqs)
    ql, qptr = _i32_array(q_lens)
    return int(load().pa_verify_step_workspace_bytes(pool, ptr, qptr, len(arr), num_heads))


def pa_verify_step(pool, seqs, q_lens, num_heads, k_new, v_new, q, out, ws, ws_bytes, stream=None,
                   slots_out=None):
    """Multi-token step; returns the new slots (int64 [sum q_lens]) when
    ``slots_out`` is given or True."""
    arr, ptr = _i64_array(seqs)
    ql, qptr = _i32_array(q_lens)
    sp = None
    if slots_out is True:
        slots_out = np.empty(int(ql.sum()), dtype=np.int64)
    if slots_out is not None:
        assert slots_out.dtype == np.int64 and slots_out.size >= int(ql.sum())
        sp = _ptr(slots_out)
    _check(load().pa_verify_step(pool, ptr, qptr, len(arr), num_heads, _addr(k_new), _addr(v_new),
                                 _addr(q), _addr(out), _addr(ws), ws_bytes, sp, _stream(stream)))
    return slots_out


def pa_prefill_workspace_bytes(pool, seqs, q_lens, num_heads):
    arr, ptr = _i64_array(seqs)
    ql, qptr = _i32_array(q_lens)
    return int(load().pa_prefill_workspace_bytes(pool, ptr, qptr, len(arr), num_heads))


def pa_prefill_chunk(pool, seqs, q_lens, num_heads, q, out, ws, ws_bytes, stream=None):
    arr, ptr = _i64_array(seqs)
    ql, qptr = _i32_array(q_lens)
    _check(load().pa_prefill_chunk(pool, ptr, qptr, len(arr), num_heads, _addr(q), _addr(out),
                                   _addr(ws), ws_bytes, _stream(stream)))


# --------------------------------------------------------------- inspection
def pa_seq_len(pool, seq):
    n = _i32()
    _check(load().pa_seq_len(pool, seq, ctypes.byref(n)))
    return n.value


def pa_block_table(pool, seq):
    n = _i32()
    _check(load().pa_block_table(pool, seq, None, 0, ctypes.byref(n)))
    out = np.empty(n.value, dtype=np.int32)
    if n.value:
        _check(load().pa_block_table(pool, seq, _ptr(out), n.value, ctypes.byref(n)))
    return out


def pa_decode_work_items(pool, seqs, num_heads, q_lens=None):
    """(pages_per_range, items [n][16] int32, tables int32) of the decode work
    list for this batch (see the header)."""
    seqs = np.ascontiguousarray(seqs, dtype=np.int64)
    ql = None if q_lens is None else np.ascontiguousarray(q_lens, dtype=np.int32)
    ppr, n_items, n_tables = _i32(), _i32(), ctypes.c_int64()
    args = (pool, _ptr(seqs), None if ql is None else _ptr(ql), len(seqs), num_heads, ctypes.byref(ppr))
    _check(load().pa_decode_work_items(*args, None, 0, ctypes.byref(n_items), None, 0, ctypes.byref(n_tables)))
    items = np.zeros((n_items.value, 16), dtype=np.int32)
    tables = np.zeros(n_tables.value, dtype=np.int32)
    _check(load().pa_decode_work_items(*args, _ptr(items), n_items.value, ctypes.byref(n_items),
                                       _ptr(tables), n_tables.value, ctypes.byref(n_tables)))
    return ppr.value, items, tables


def pa_refcount(pool, block):
    rc = _i32()
    _check(load().pa_refcount(pool, block, ctypes.byref(rc)))
    return rc.value


def pa_stats(pool):
    st = pa_pool_stats()
    _check(load().pa_stats(pool, ctypes.byref(st)))
    return {name: getattr(st, name) for name, _ in pa_pool_stats._fields_}


def pa_validate(pool):
    _check(load().pa_validate(pool))


def pa_sequences(pool):
    n = _i32()
    _check(load().pa_sequences(pool, None, 0, ctypes.byref(n)))
    out = np.empty(n.value, dtype=np.int64)
    if n.value:
        _check(load().pa_sequences(pool, _ptr(out), n.value, ctypes.byref(n)))
    return out


def pa_last_error():
    return load().pa_last_error().decode("utf-8", "replace")


def pa_timing_enable(on=True):
    _check(load().pa_timing_enable(1 if on else 0))


def pa_timing_select(kernels=None):
    """Time only the listed kernel families (PA_KERNEL_*); None = all."""
    mask = 0xFFFFFFFF if kernels is None else sum(1 << int(k) for k in kernels)
    _check(load().pa_timing_select(mask))


def pa_timing_reset():
    _check(load().pa_timing_reset())


def pa_timing_read(kernel):
    ms = ctypes.c_double()
    n = _i64()
    _check(load().pa_timing_read(kernel, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def pa_timing_samples(kernel):
    """Per-launch durations (ms, launch order) of one kernel family since the last reset."""
    n = _i64()
    _check(load().pa_timing_samples(kernel, None, 0, ctypes.byref(n)))
    buf = (ctypes.c_float * max(n.value, 1))()
    _check(load().pa_timing_samples(kernel, buf, n.value, ctypes.byref(n)))
    return [float(buf[i]) for i in range(n.value)]
