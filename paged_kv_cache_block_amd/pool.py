"""DevicePool: a paged KV pool whose K/V memory is a pair of torch tensors.

Convenience layer over :mod:`paged_kv_cache_block_amd.abi`: torch allocates
the pools, the decode / prefill workspaces and the device copy of the slot
mapping; everything else (bookkeeping, cache writes, attention) is a call
into libpagedattn.so on the current torch stream.
"""

from __future__ import annotations

import numpy as np

from . import abi

_DTYPES = {"f32": abi.PA_DTYPE_F32, "bf16": abi.PA_DTYPE_BF16, "i8": abi.PA_DTYPE_I8,
           "fp8": abi.PA_DTYPE_FP8}


def _torch():
    import torch
    return torch


class DevicePool:
    """One pool of ``num_blocks`` blocks; K and V live on ``device``.

    ``dtype`` is "bf16", "f32", "i8" or "fp8" (int8 or E4M3 codes with one
    fp32 scale per (token, KV head) row; queries, outputs and new rows are
    then bf16, and ``k`` / ``v`` are raw byte tensors ``[num_blocks,
    num_kv_heads, page_bytes]`` in the library's 8-bit page layout).  bf16
    ``k`` is ``[num_blocks, num_kv_heads, block_size * head_dim]`` in the
    library's K page order, fp32 ``k`` ``[num_blocks, num_kv_heads,
    block_size, head_dim]``; ``v`` of both is ``[num_blocks, num_kv_heads,
    head_dim, block_size]``.
    With ``metadata_only=True`` no device memory is allocated and only the
    bookkeeping calls work (usable on a machine without a GPU).
    """

    def __init__(self, num_blocks, block_size, num_kv_heads, head_dim, dtype="bf16",
                 allocation_order=None, device="cuda", metadata_only=False):
        self.num_blocks, self.block_size = num_blocks, block_size
        self.num_kv_heads, self.head_dim = num_kv_heads, head_dim
        self.dtype = dtype
        self.desc = abi.make_desc(num_blocks, block_size, num_kv_heads, head_dim, _DTYPES[dtype])
        self.k = self.v = None
        self._ws = None
        self.handle = None
        if not metadata_only:
            torch = _torch()
            if dtype in ("i8", "fp8"):
                page = block_size * head_dim + 4 * block_size
                shape_k = shape_v = (num_blocks, num_kv_heads, page)
                tdt = torch.uint8
            else:
                tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
                shape_k = ((num_blocks, num_kv_heads, block_size * head_dim) if dtype == "bf16"
                           else (num_blocks, num_kv_heads, block_size, head_dim))
                shape_v = (num_blocks, num_kv_heads, head_dim, block_size)
            self.k = torch.zeros(shape_k, dtype=tdt, device=device)
            self.v = torch.zeros(shape_v, dtype=tdt, device=device)
            assert self.k.numel() * self.k.element_size() == abi.pa_pool_bytes(self.desc)
        self.handle = abi.pa_pool_create(self.desc, allocation_order, self.k, self.v)

    @property
    def io_dtype(self):
        """torch dtype of queries, outputs and new K/V rows."""
        torch = _torch()
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    # ------------------------------------------------------------ lifetime
    def close(self):
        if self.handle is not None:
            abi.pa_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------ metadata
    def create(self, seq):
        abi.pa_seq_create(self.handle, seq)

    def append(self, seq, n_tokens):
        return abi.pa_append(self.handle, seq, n_tokens)

    def append_batch(self, seqs, n_tokens, slots_out=None):
        return abi.pa_append_batch(self.handle, seqs, n_tokens, slots_out)

    def share(self, src, dst, prefix_tokens):
        abi.pa_share(self.handle, src, dst, prefix_tokens)

    def fork(self, src, dst):
        abi.pa_fork(self.handle, src, dst)

    def release(self, seq):
        abi.pa_release(self.handle, seq)

    def set_window(self, seq, sink_tokens, recent_tokens):
        abi.pa_seq_set_window(self.handle, seq, sink_tokens, recent_tokens)

    def truncate(self, seq, new_length):
        abi.pa_truncate(self.handle, seq, new_length)

    # ------------------------------------------------------------ prefix cache
    def prefix_lookup(self, tokens, scope, revision):
        return abi.pa_prefix_lookup(self.handle, scope, revision, tokens)

    def prefix_attach(self, seq, tokens, scope, revision):
        return abi.pa_prefix_attach(self.handle, seq, scope, revision, tokens)

    def prefix_register(self, seq, tokens, scope, revision):
        return abi.pa_prefix_register(self.handle, seq, scope, revision, tokens)

    def prefix_clear(self):
        return abi.pa_prefix_clear(self.handle)

    def prefix_entries(self):
        return abi.pa_prefix_entries(self.handle)

    def pending_copies(self):
        return abi.pa_pending_copies(self.handle)

    def seq_len(self, seq):
        return abi.pa_seq_len(self.handle, seq)

    def block_table(self, seq):
        return abi.pa_block_table(self.handle, seq)

    def decode_work_items(self, seqs, num_heads, q_lens=None):
        """(pages per range, work items [n][16], visited-page tables) of the
        decode work list for this batch (pa_decode_work_items)."""
        return abi.pa_decode_work_items(self.handle, seqs, num_heads, q_lens)

    def refcount(self, block):
        return abi.pa_refcount(self.handle, block)

    def stats(self):
        return abi.pa_stats(self.handle)

    def validate(self):
        abi.pa_validate(self.handle)

    def sequences(self):
        return abi.pa_sequences(self.handle)

    # ------------------------------------------------------------ device work
    @staticmethod
    def _stream(stream):
        if stream is not None:
            return stream
        return _torch().cuda.current_stream().cuda_stream

    def flush(self, stream=None):
        abi.pa_flush_copies(self.handle, self._stream(stream))

    def _rows(self, t, rows, heads, name):
        """``t`` must be a contiguous device tensor [rows, heads, head_dim] of
        the pool's input dtype: the kernels read and write exactly that many
        bytes through its pointer."""
        torch = _torch()
        if self.k is None:  # metadata-only pool: the library rejects the call itself
            return
        ok = (torch.is_tensor(t) and t.device == self.k.device and t.dtype == self.io_dtype
              and t.is_contiguous() and tuple(t.shape) == (rows, heads, self.head_dim))
        if not ok:
            got = (tuple(t.shape), t.dtype, str(t.device), t.is_contiguous()) if torch.is_tensor(t) else type(t)
            raise ValueError(f"{name} must be a contiguous {self.io_dtype} tensor of shape "
                             f"{(rows, heads, self.head_dim)} on {self.k.device}; got {got}")

    def _queries(self, q, out, rows):
        if not _torch().is_tensor(q) or q.dim() != 3:
            raise ValueError("q must be a [rows, num_heads, head_dim] tensor")
        heads = int(q.shape[1])
        self._rows(q, rows, heads, "q")
        if out is None:
            out = _torch().empty_like(q)
        self._rows(out, rows, heads, "out")
        return heads, out

    def write(self, slots, k_new, v_new, stream=None):
        """Store rows ``k_new[i], v_new[i]`` ([n, Hkv, D] device tensors) at ``slots``."""
        torch = _torch()
        if not torch.is_tensor(slots) or slots.device.type != "cuda":
            slots = torch.as_tensor(np.asarray(slots, dtype=np.int64)).to(self.k.device, non_blocking=False)
        if slots.dtype != torch.int64 or not slots.is_contiguous():
            raise ValueError("slots must be a contiguous int64 tensor")
        n = int(slots.numel())
        self._rows(k_new, n, self.num_kv_heads, "k_new")
        self._rows(v_new, n, self.num_kv_heads, "v_new")
        abi.pa_reshape_and_cache(self.handle, k_new, v_new, slots, n, self._stream(stream))
        return slots

    def set_slot_checks(self, on, stream=None):
        """Debug checks of ``write`` (pa_pool_set_slot_checks): bad or
        repeated slots are rejected before anything is written."""
        abi.pa_pool_set_slot_checks(self.handle, on, self._stream(stream))

    def workspace(self, nbytes):
        torch = _torch()
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.k.device)
            assert self._ws.data_ptr() % 256 == 0
        return self._ws

    def decode(self, seqs, q, out=None, stream=None, ws=None):
        """One query row per sequence: ``q`` [B, Hq, D] -> ``out`` [B, Hq, D]."""
        num_heads, out = self._queries(q, out, len(seqs))
        need = abi.pa_decode_workspace_bytes(self.handle, seqs, num_heads)
        if need == 0:
            # Invalid batch: let the call itself report why.
            need = 256
        if ws is None:
            ws = self.workspace(need)
        abi.pa_decode(self.handle, seqs, num_heads, q, out, ws, ws.numel(), self._stream(stream))
        return out

    def decode_step(self, seqs, k_new, v_new, q, out=None, stream=None, ws=None):
        """Append one token per sequence, store its K/V, decode over the caches.

        Returns ``(out, slots)``."""
        num_heads, out = self._queries(q, out, len(seqs))
        self._rows(k_new, len(seqs), self.num_kv_heads, "k_new")
        self._rows(v_new, len(seqs), self.num_kv_heads, "v_new")
        need = abi.pa_decode_step_workspace_bytes(self.handle, seqs, num_heads) or 256
        if ws is None:
            ws = self.workspace(need)
        slots = abi.pa_decode_step(self.handle, seqs, num_heads, k_new, v_new, q, out, ws, ws.numel(),
                                   self._stream(stream), slots_out=True)
        return out, slots

    def decode_step_noalloc(self, seqs, k_new, v_new, q, out, stream=None):
        """decode_step with the library's static scratch as its workspace
        (pa_decode_step_noalloc: no device or pinned allocation in the call;
        ``out`` must be given).  Returns ``(out, slots)``."""
        if out is None:
            raise ValueError("decode_step_noalloc needs a caller-allocated out")
        num_heads, out = self._queries(q, out, len(seqs))
        self._rows(k_new, len(seqs), self.num_kv_heads, "k_new")
        self._rows(v_new, len(seqs), self.num_kv_heads, "v_new")
        slots = abi.pa_decode_step_noalloc(self.handle, seqs, num_heads, k_new, v_new, q, out,
                                           self._stream(stream), slots_out=True)
        return out, slots

    def verify_step(self, seqs, q_lens, k_new, v_new, q, out=None, stream=None, ws=None):
        """Append ``q_lens[b]`` tokens per sequence, store their K/V rows
        ([sum q_lens, Hkv, D]) and attend causally for those rows (``q``
        [sum q_lens, Hq, D]).  Returns ``(out, slots)``."""
        rows = int(np.sum(np.asarray(q_lens, dtype=np.int64)))
        num_heads, out = self._queries(q, out, rows)
        self._rows(k_new, rows, self.num_kv_heads, "k_new")
        self._rows(v_new, rows, self.num_kv_heads, "v_new")
        need = abi.pa_verify_step_workspace_bytes(self.handle, seqs, q_lens, num_heads) or 256
        if ws is None:
            ws = self.workspace(need)
        slots = abi.pa_verify_step(self.handle, seqs, q_lens, num_heads, k_new, v_new, q, out, ws,
                                   ws.numel(), self._stream(stream), slots_out=True)
        return out, slots

    def prefill(self, seqs, q_lens, q, out=None, stream=None, ws=None):
        """Last ``q_lens[b]`` positions of each sequence: ``q`` [sum q_lens, Hq, D]."""
        rows = int(np.sum(np.asarray(q_lens, dtype=np.int64)))
        num_heads, out = self._queries(q, out, rows)
        need = abi.pa_prefill_workspace_bytes(self.handle, seqs, q_lens, num_heads) or 256
        if ws is None:
            ws = self.workspace(need)
        abi.pa_prefill_chunk(self.handle, seqs, q_lens, num_heads, q, out, ws, ws.numel(),
                             self._stream(stream))
        return out
