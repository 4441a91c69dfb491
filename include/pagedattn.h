/*
 * pagedattn.h -- C ABI of libpagedattn.so: paged attention over a refcounted
 * pool of KV blocks, for AMD Instinct MI355X (gfx950).
 *
 * Sources this interface follows (cited by page title and section):
 *   [KVPool]    abhik.ai "examples/pagedattention.py", class KVPool and its
 *               regions physical_pool, logical_address, append_or_allocate,
 *               fork_prefix, copy_on_write, paged_attention, release_sequence.
 *   [PagedPool] vladkulikov.com notebook "Модуль 10. KV-кэши и эффективный
 *               инференс", class PagedKVPool (preflighted append, share_prefix,
 *               release, fill accounting, validate) and its negative tests.
 *   [ferrum]    docs.rs ferrum-kv 0.4.0 src/attention.rs, paged_attention
 *               (GQA grouping, 1/sqrt(head_dim) scale, causal mask) and
 *               PagedKvCacheManager::write_kv as its caller uses it.
 *   [lecture19] CMU 11-667 lecture 19 infer_world.py, section 3 (online
 *               softmax statistics, tiled attention).
 *   [KVprefix]  vladkulikov.com notebook "Модуль 10", the prefix-caching
 *               cell (prefix_key, run_prefix_trace) and its key-identity
 *               checks.
 *   [KVwindow]  vladkulikov.com notebook "Модуль 10", the eviction cell
 *               (streaming_keep_indices) and the explicit window caches
 *               (window, truncate).
 *   [KVquant]   vladkulikov.com notebook "Модуль 10", the KV-compression
 *               experiment (per-row absmax codes, fake_quantize_rows, and
 *               the packed size of codes plus one fp32 scale per row).
 *
 * Conventions for every call
 *   - Sequence ids are arbitrary int64 values chosen by the caller.
 *   - "host" pointers are ordinary CPU memory read or written before the call
 *     returns; "device" pointers are GPU memory owned by the caller (e.g.
 *     torch tensors).  The library never frees caller memory.  A pool object
 *     owns only host metadata plus a few pinned host staging buffers.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Device work is enqueued on it and the call returns without waiting,
 *     except where stated.  All device calls on one pool must use one stream
 *     (or be ordered by the caller): pending copy-on-write copies are
 *     flushed onto whichever stream the next device call names.
 *   - Every call validates all arguments first and, where it allocates
 *     blocks, preflights the block count; on any error the pool is unchanged
 *     (strong guarantee, [KVPool] append/_private_tail, [PagedPool] append and
 *     its "OOM leaves the snapshot unchanged" negative test).  The message of
 *     the last error on the calling thread is returned by pa_last_error().
 *   - A pool is not thread-safe.
 *
 * Device layouts (element size 4 for PA_DTYPE_F32, 2 for BF16):
 *   K pool  [num_blocks][num_kv_heads][page of block_size * head_dim values]
 *   V pool  [num_blocks][num_kv_heads][head_dim][block_size]
 *   (one (block, KV head) page of V is stored transposed, head_dim rows of
 *    block_size tokens, so that the P.V contraction over tokens reads
 *    contiguous memory.)  A K page of PA_DTYPE_F32, or of BF16 with
 *   block_size % 16 != 0 or head_dim % 32 != 0, is row-major
 *   [block_size][head_dim].  Other BF16 K pages are in the order of the
 *   decode kernel's operands: in each 16-token tile, the 8 values
 *   d = 32 j + 8 grp .. +7 of token t sit at element
 *     (t / 16) * 16 * head_dim + (j * 64 + grp * 16 + t % 16) * 8 + d % 8,
 *   so one 64-lane load of 16 bytes per lane reads 1 KB of consecutive
 *   memory.
 *   Both pools must be 16-byte aligned.  The layout is a physical choice:
 *   the logical K/V row of token p of a sequence is the slot
 *   table[p / block_size] * block_size + p % block_size ([KVPool]
 *   logical_address), whatever the layout.
 *   q / out for decode   [B][num_heads][head_dim]
 *   q / out for prefill  [sum(q_lens)][num_heads][head_dim] (sequence-major,
 *                        [ferrum] "[q_tokens, num_heads, head_dim]")
 *   k_new / v_new        [n][num_kv_heads][head_dim]
 *   q, out, k_new and v_new use the pool dtype (bf16 for PA_DTYPE_I8 and
 *   PA_DTYPE_FP8);
 *   accumulation is fp32.
 *
 * PA_DTYPE_I8 pools ([KVquant]) store each (token, KV head) row of K and of
 * V as head_dim int8 codes plus one fp32 scale; the row reads back as
 * code * scale.  The cache writes derive them from the bf16 row x, in
 * float64: scale = max|x| / 127 (1 for an all-zero row), code =
 * x / scale rounded to nearest, ties to even, clipped to [-127, 127]; the
 * stored scale is that float64 value rounded to fp32.  Requires block_size
 * and head_dim to be multiples of 16.  One page (block, KV head) of either
 * pool is page_bytes = block_size * head_dim + 4 * block_size bytes, the
 * codes (block_size * head_dim bytes, in 16-token tiles of 16 * head_dim
 * bytes) then the block_size fp32 scales:
 *   K codes  with head_dim % 64 == 0: with span = head_dim / 4, the code of
 *            token t, dim d (grp = d / span, c = d % span) sits at byte
 *              (t / 16) * 16 * head_dim + ((c / 16) * 64 + grp * 16 + t % 16)
 *              * 16 + c % 16;
 *            other head_dims: row-major [block_size][head_dim].
 *   V codes  MFMA operand order: in each 16-token tile, row r = (t % 16) / 4
 *            * 16 + d % 16 holds head_dim / 4 codes, byte c = (d / 16) * 4 +
 *            t % 4 of the row; with head_dim % 64 == 0 the code sits at
 *              (t / 16) * 16 * head_dim + ((c / 16) * 64 + r) * 16 + c % 16,
 *            otherwise at (t / 16) * 16 * head_dim + r * (head_dim / 4) + c.
 *   Either way one 64-lane load of 16 bytes per lane reads 1 KB of
 *   consecutive codes in the decode kernel's operand order.
 *   pool bytes = num_blocks * num_kv_heads * page_bytes (each of K, V).
 *
 * PA_DTYPE_FP8 pools hold the same rows and pages with 8-bit float codes
 * instead of integers (an extension of [KVquant]'s scheme): scale = max|x| /
 * 448 in float64 (1 for an all-zero row), code = the E4M3 value nearest to
 * x / scale (float64; ties to the even code, magnitudes above 448 to 448; a
 * zero is 0x00).  E4M3 here: bit 7 sign, bits 6..3 exponent with bias 7,
 * bits 2..0 mantissa; exponent 0 holds the subnormals m * 2^-9, otherwise
 * (1 + m / 8) * 2^(e - 7); no infinities, the magnitude 0x7F is not a number
 * and never written, 0x7E = 448 is the largest.  A row reads back as
 * value(code) * scale, with the scale stored as fp32.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_pool pa_pool; /* opaque; owns host metadata only */

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1,   /* bad size, pointer, prefix, q_len, workspace, ... */
  PA_ERR_UNKNOWN_SEQ = -2,   /* id not live: never created or already released */
  PA_ERR_SEQ_EXISTS = -3,    /* id already live */
  PA_ERR_OUT_OF_BLOCKS = -4, /* preflight: the pool cannot supply the blocks */
  PA_ERR_DEVICE = -5         /* a HIP call failed (message in pa_last_error) */
} pa_status;

typedef enum {
  PA_DTYPE_F32 = 0,  /* fp32 K/V, q, out */
  PA_DTYPE_BF16 = 1, /* bf16 K/V, q, out */
  PA_DTYPE_I8 = 2,   /* int8 K/V codes + fp32 row scales; bf16 q, out, new rows */
  PA_DTYPE_FP8 = 3   /* E4M3 K/V codes + fp32 row scales; bf16 q, out, new rows */
} pa_dtype;

typedef struct {
  int32_t num_blocks;   /* physical blocks in the pool, > 0 */
  int32_t block_size;   /* token slots per block, > 0 */
  int32_t num_kv_heads; /* KV heads stored per token, > 0 */
  int32_t head_dim;     /* values per head, 1..512 */
  int32_t dtype;        /* pa_dtype of K, V, q and out */
} pa_pool_desc;

/* Accounting of [PagedPool] (allocated_blocks ... sharing_savings_tokens).
 * A block's fill is the largest number of live slots any sequence holding it
 * uses; payload sums fills over referenced blocks; capacity is
 * allocated * block_size; waste = capacity - payload; logical sums sequence
 * lengths; savings = logical - payload. */
typedef struct {
  int64_t allocated_blocks, free_blocks, physical_capacity_tokens,
      physical_payload_tokens, logical_tokens, internal_waste_tokens,
      sharing_savings_tokens;
} pa_pool_stats;

/* ---------------------------------------------------------------- pool --- */

/* Bytes of ONE of the K / V pools for `desc`:
 * num_blocks * num_kv_heads * block_size * head_dim * element size, or for
 * PA_DTYPE_I8 and PA_DTYPE_FP8 num_blocks * num_kv_heads * (block_size *
 * head_dim + 4 * block_size).  Returns 0 for an invalid descriptor
 * (including an I8 or FP8 descriptor whose block_size or head_dim is not a
 * multiple of 16). */
size_t pa_pool_bytes(const pa_pool_desc* desc);

/* Create a pool over caller-allocated device pools ([KVPool] physical_pool).
 * allocation_order: host [num_blocks], a full permutation of 0..num_blocks-1
 *   giving the order in which free blocks are handed out (the free block of
 *   lowest rank is taken next, [KVPool] _allocate), or NULL for 0,1,2,...
 * k_pool, v_pool: device, pa_pool_bytes(desc) bytes each, laid out as in the
 *   header comment; both NULL gives a metadata-only pool (every device call
 *   on it fails with PA_ERR_INVALID_ARG).  The caller keeps ownership and
 *   must keep them alive until pa_pool_destroy.
 * out: receives the new pool.
 * A pool with device memory also reserves its ring of 4 pinned host staging
 *   buffers here (through which plans cross to the device), each of
 *   min(8 * num_blocks + 256 KiB, 8 MiB) bytes, so the attention calls
 *   allocate nothing while their plans fit (pa_pool_reserve_staging).
 * Errors: PA_ERR_INVALID_ARG for a bad descriptor, a non-permutation order,
 *   exactly one NULL pool pointer, misaligned pools or a NULL `out`;
 *   PA_ERR_DEVICE if the staging buffers cannot be allocated. */
pa_status pa_pool_create(const pa_pool_desc* desc, const int32_t* allocation_order,
                         void* k_pool, void* v_pool, pa_pool** out);

/* Grow each of the pool's 4 pinned staging buffers to at least plan_bytes
 * (buffers still in use by enqueued work are waited for first; none
 * shrinks).  A call whose plan exceeds the reserved size grows the ring
 * inside that call (pinned allocation), except pa_decode_step_noalloc,
 * which fails instead.  A plan is at most the metadata part of the
 * workspace the *_workspace_bytes calls return, so reserving that much is
 * always enough.  reserved: host, may be NULL; receives the size now
 * reserved per buffer.  Host-side; allocates pinned host memory.
 * Errors: PA_ERR_INVALID_ARG (NULL or metadata-only pool, plan_bytes above
 *   4 GiB), PA_ERR_DEVICE. */
pa_status pa_pool_reserve_staging(pa_pool* pool, size_t plan_bytes, size_t* reserved);

/* Free the pool's host metadata and staging buffers (waits for the pool's
 * own pending uploads).  NULL is ignored. */
void pa_pool_destroy(pa_pool* pool);

/* New empty sequence, length 0; no block is reserved ([KVPool] create,
 * [PagedPool] create).  Errors: PA_ERR_SEQ_EXISTS. */
pa_status pa_seq_create(pa_pool* pool, int64_t seq);

/* Append n_tokens >= 0 logical tokens to `seq` ([PagedPool] append; [KVPool]
 * append_or_allocate and copy_on_write).
 * Preflight: needs = (1 if the tail block is partially filled and shared)
 *   + ceil(max(0, n_tokens - room_in_tail) / block_size); if needs exceeds
 *   the free blocks, PA_ERR_OUT_OF_BLOCKS and nothing changes.
 * Then a shared partial tail is replaced by a fresh block and a whole-block
 *   copy old -> new is recorded as pending (executed on the device by the
 *   next device call on this pool, or pa_flush_copies), the tail is filled
 *   and whole new blocks are taken in allocation order.
 * slots_out: host [n_tokens] (may be NULL when n_tokens == 0); receives the
 *   slot of each new position p = old_len .. old_len+n_tokens-1, i.e.
 *   table[p / block_size] * block_size + p % block_size.  Pass them (on the
 *   device) to pa_reshape_and_cache.
 * This call is host-only: it launches nothing.  Hazard of the deferred
 *   copy: until the next device call on this pool (or pa_flush_copies) has
 *   been enqueued, the new tail block does not hold the old tail's rows yet,
 *   and the old block must still hold them.  So the caller must not write
 *   the pool's device memory by other means (a torch copy into the pools,
 *   another library) before that call: flush first, on the same stream.
 * Errors: PA_ERR_UNKNOWN_SEQ, PA_ERR_INVALID_ARG (n_tokens < 0, NULL
 *   slots_out with n_tokens > 0), PA_ERR_OUT_OF_BLOCKS. */
pa_status pa_append(pa_pool* pool, int64_t seq, int32_t n_tokens, int64_t* slots_out);

/* pa_append(pool, seqs[i], n_tokens[i], ...) for i = 0 .. count-1, in order
 * (a decode step appends one token to every sequence of the batch), with the
 * slots of all appends concatenated in slots_out (host [sum n_tokens]).
 * All or nothing: if any append fails, the earlier appends of the batch are
 * undone (tables, lengths, refcounts, free blocks and pending copies are as
 * before the call) and that append's status is returned.  Host-only.
 * Errors: as pa_append; PA_ERR_INVALID_ARG for count < 0 or NULL arrays. */
pa_status pa_append_batch(pa_pool* pool, const int64_t* seqs, const int32_t* n_tokens,
                          int32_t count, int64_t* slots_out);

/* New sequence `dst` holding the first ceil(prefix_tokens / block_size)
 * blocks of `src` with every refcount + 1 and length prefix_tokens
 * ([PagedPool] share_prefix).  Host-only.
 * Errors: PA_ERR_UNKNOWN_SEQ (src), PA_ERR_SEQ_EXISTS (dst),
 *   PA_ERR_INVALID_ARG (prefix_tokens < 0, > length of src, or before the
 *   end of pages src's window released). */
pa_status pa_share(pa_pool* pool, int64_t src, int64_t dst, int32_t prefix_tokens);

/* pa_share(pool, src, dst, length of src): the child holds the parent's whole
 * table ([KVPool] fork_prefix).  Host-only.  Errors as pa_share. */
pa_status pa_fork(pa_pool* pool, int64_t src, int64_t dst);

/* Drop one reference to each block of `seq` and forget it; blocks whose
 * refcount reaches 0 become free ([KVPool] release_sequence, [PagedPool]
 * release).  A second release of the same id is PA_ERR_UNKNOWN_SEQ.
 * Host-only; device contents are left as they are. */
pa_status pa_release(pa_pool* pool, int64_t seq);

/* ------------------------------------------------------ windows, rollback --- */
/* Sliding window with attention sinks ([KVwindow]).  After this call every
 * query row of `seq` (position p, causal limit p + 1) sees the positions
 * streaming_keep_indices(p + 1, sink_tokens + recent_tokens, sink_tokens)
 * keeps: all of [0, p] while p + 1 <= sink_tokens + recent_tokens, else
 * [0, sink_tokens) and [p + 1 - recent_tokens, p].  Each later append of n
 * tokens at old length L0 releases (refcount - 1, the table entry becomes
 * -1) the pages lying wholly after the sink pages and before position
 * L0 + 1 - recent_tokens (the window of its first appended row), never a
 * page holding an appended row; the decode kernels skip the pages no row
 * sees.  Released positions stay counted in the length and are gone:
 * a row sees the kept positions that are still resident.  fork / share
 * copy the window and the released entries.  Host-only.
 * Errors: PA_ERR_UNKNOWN_SEQ; PA_ERR_INVALID_ARG unless sink_tokens >= 0,
 *   recent_tokens >= 0 and 1 <= sink_tokens + recent_tokens. */
pa_status pa_seq_set_window(pa_pool* pool, int64_t seq, int32_t sink_tokens, int32_t recent_tokens);

/* Roll `seq` back to new_length (speculative tokens rejected): positions
 * [new_length, length) are dropped and pages past ceil(new_length /
 * block_size) released.  new_length may not fall before the first position
 * after the last released page ([KVwindow] rollback cannot bring evicted
 * tokens back).  A later append into a shared partial tail copies it first.
 * Host-only.  Errors: PA_ERR_UNKNOWN_SEQ, PA_ERR_INVALID_ARG. */
pa_status pa_truncate(pa_pool* pool, int64_t seq, int32_t new_length);

/* ---------------------------------------------------------- prefix cache --- */
/* Prefix-hash block reuse ([KVprefix]).  Each pool owns one cache.  A key
 * exists only at a complete block boundary end (a multiple of block_size)
 * and is (scope, revision, token ids [0, end)): equal block contents after a
 * different context, or under another scope or model revision, are
 * different keys.  A cached key maps to the physical block holding tokens
 * [end - block_size, end) and holds one reference to it (a pin: the block
 * outlives the sequences that wrote it, refcounts include pins, and a block
 * only pins hold counts as capacity, not payload, in pa_stats).  The cache
 * has no eviction ([KVprefix] has none); pa_prefix_clear drops every key.
 * scope, revision: NUL-terminated byte strings; tokens: host int32 ids.
 * All calls are host-only. */

/* Hit of tokens[0 .. n_tokens): the largest h (a multiple of block_size) such
 * that every complete-block key up to h is cached.  Nothing changes. */
pa_status pa_prefix_lookup(const pa_pool* pool, const char* scope, const char* revision,
                           const int32_t* tokens, int32_t n_tokens, int32_t* hit_tokens);

/* New sequence `seq` holding the cached blocks of its hit h (refcount + 1
 * each, like pa_share) with length h; *hit_tokens receives h.  The caller
 * then appends and stores the remaining n_tokens - h positions.
 * Errors: PA_ERR_SEQ_EXISTS, PA_ERR_INVALID_ARG (NULL pointers, n < 0). */
pa_status pa_prefix_attach(pa_pool* pool, int64_t seq, const char* scope, const char* revision,
                           const int32_t* tokens, int32_t n_tokens, int32_t* hit_tokens);

/* Add the keys of the complete blocks of `seq`'s first n_tokens positions,
 * whose token ids are tokens[0 .. n_tokens) and whose K/V the caller has
 * stored (or enqueued).  A key already cached keeps its block; each new key
 * pins seq's block.  *added_blocks (may be NULL) receives the new key count.
 * Errors: PA_ERR_UNKNOWN_SEQ, PA_ERR_INVALID_ARG (n_tokens > length(seq)). */
pa_status pa_prefix_register(pa_pool* pool, int64_t seq, const char* scope, const char* revision,
                             const int32_t* tokens, int32_t n_tokens, int32_t* added_blocks);

/* Drop every key and its pin (blocks no table holds become free);
 * *dropped_entries (may be NULL) receives the number of keys. */
pa_status pa_prefix_clear(pa_pool* pool, int32_t* dropped_entries);

/* Number of cached keys (= pinned block references). */
pa_status pa_prefix_entries(const pa_pool* pool, int64_t* entries);

/* Pending copy-on-write copies, oldest first, as (src, dst) block pairs.
 * pairs_out: host [2 * cap]; *n receives the number pending (may exceed cap;
 * then only the first cap are written).  Errors: PA_ERR_INVALID_ARG. */
pa_status pa_pending_copies(const pa_pool* pool, int32_t* pairs_out, int32_t cap, int32_t* n);

/* Enqueue the pending whole-block copies (K and V, every head) on `stream`
 * in recording order, then clear the list.  Called implicitly at the start
 * of pa_reshape_and_cache, pa_decode and pa_prefill_chunk.
 * Errors: PA_ERR_INVALID_ARG (metadata-only pool), PA_ERR_DEVICE. */
pa_status pa_flush_copies(pa_pool* pool, void* stream);

/* Write new K/V rows into their slots ([KVPool] append stores the row at
 * (table[p / block_size], p % block_size); ferrum's write_kv):
 *   K page (slot / bs, h), token slot % bs   <- k_new[i][h][:]
 *   Vpool[slot / bs][h][:][slot % bs]        <- v_new[i][h][:]   for i < n, every h,
 * each K value at its place in the K page order of the header comment.
 * k_new, v_new: device [n][num_kv_heads][head_dim]; slots: device int64 [n].
 * An I8 or FP8 pool stores each row's codes and scale instead ([KVquant];
 * the layout and rounding are in the header comment).
 * Without slot checks (the default) a slot outside [0, num_blocks *
 * block_size) is skipped and two rows naming one slot race; with them
 * (pa_pool_set_slot_checks) the call is rejected first.  Pending copies are
 * flushed first on `stream`.
 * Errors: PA_ERR_INVALID_ARG (NULL pointers with n > 0, n < 0,
 *   metadata-only pool; with slot checks on, a bad slot), PA_ERR_DEVICE. */
pa_status pa_reshape_and_cache(pa_pool* pool, const void* k_new, const void* v_new,
                               const int64_t* slots, int32_t n, void* stream);

/* Debug checks of this pool's pa_reshape_and_cache calls, off by default
 * (validate before mutate, as [PagedPool]'s negative tests ask of every
 * operation).  When on, each call first checks on the device, before it
 * writes anything, that every slot lies in [0, num_blocks * block_size) and
 * that no two rows of the call name one slot; it waits for that check
 * (synchronizing `stream`) and on failure returns PA_ERR_INVALID_ARG naming
 * an offending row and its slot, with the pool's memory and pending copies
 * untouched.  Turning the checks on allocates 4 bytes of device memory per
 * slot, zeroed on `stream`; turning them off (or pa_pool_destroy) frees it
 * after waiting for the device.  The fused steps compute their slots
 * themselves and are not checked.
 * Errors: PA_ERR_INVALID_ARG (NULL or metadata-only pool), PA_ERR_DEVICE. */
pa_status pa_pool_set_slot_checks(pa_pool* pool, int on, void* stream);

/* ------------------------------------------------------------ attention --- */

/* Workspace bytes pa_decode needs for this batch (a device buffer the caller
 * allocates; it holds the uploaded block tables, the work list and split-K
 * partial results).  0 if the arguments are invalid. */
size_t pa_decode_workspace_bytes(const pa_pool* pool, const int64_t* seqs, int32_t B,
                                 int32_t num_heads);

/* Decode attention: one query row per sequence attends over every cached
 * token of that sequence ([KVPool] paged_attention: the next position sees
 * the whole cache; [ferrum] paged_attention with q_tokens = 1):
 *   for b < B, h < num_heads, with L = length(seqs[b]), G = num_heads /
 *   num_kv_heads, g = h / G, K_j / V_j = the rows of token j gathered
 *   through the block table:
 *     s_j = (q[b][h] . K_j[g]) / sqrt(head_dim),  j < L
 *     out[b][h] = sum_j softmax(s)_j V_j[g]
 * Long sequences are split into page ranges whose partial (max, sum, acc)
 * are merged by log-sum-exp ([lecture19] online_softmax_stats applied
 * across ranges).
 * On an I8 or FP8 pool K_j and V_j are the rows read back (value(code) * scale).
 * seqs: host [B] live ids (duplicates allowed); q, out: device
 *   [B][num_heads][head_dim] in the pool dtype; ws: device, at least
 *   pa_decode_workspace_bytes(...) bytes, 256-byte aligned, owned by the
 *   caller and overwritten by this call (do not reuse it for another call
 *   until this one has finished on `stream`).
 * A windowed sequence's row sees its window (pa_seq_set_window).
 * Errors: PA_ERR_UNKNOWN_SEQ, PA_ERR_INVALID_ARG (B <= 0, num_heads not a
 *   positive multiple of num_kv_heads, a sequence of length 0 ([ferrum]
 *   "kv_len must be positive"), a query row in a released page, small or
 *   misaligned ws, NULL pointers, metadata-only pool), PA_ERR_DEVICE. */
pa_status pa_decode(pa_pool* pool, const int64_t* seqs, int32_t B, int32_t num_heads,
                    const void* q, void* out, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes pa_decode_step needs for this batch (sized for the lengths
 * after its append).  0 if the arguments are invalid. */
size_t pa_decode_step_workspace_bytes(const pa_pool* pool, const int64_t* seqs, int32_t B,
                                      int32_t num_heads);

/* One decode step of one layer, fused: the append of one token to every
 * sequence of the batch (pa_append_batch with n_tokens = 1 each, all or
 * nothing), the store of that token's K/V rows into their slots
 * (pa_reshape_and_cache) and decode attention of q over every cached token,
 * the new one included (pa_decode).  The plan and the slots cross to the
 * device in one upload and one kernel both copies the plan and stores the
 * new rows, so a step costs that kernel, the decode kernel and the merge.
 * k_new, v_new: device [B][num_kv_heads][head_dim]; q, out as pa_decode;
 * ws: at least pa_decode_step_workspace_bytes(...) bytes, 256-byte aligned;
 * slots_out: host [B] or NULL, receives the new slots.
 * Errors: as pa_decode and pa_append_batch; a too-small workspace or an
 *   exhausted pool is reported before anything changes.  On PA_ERR_DEVICE
 *   the append is kept (the device work could not be enqueued). */
pa_status pa_decode_step(pa_pool* pool, const int64_t* seqs, int32_t B, int32_t num_heads,
                         const void* k_new, const void* v_new, const void* q, void* out, void* ws,
                         size_t ws_bytes, int64_t* slots_out, void* stream);

/* pa_decode_step for callers that cannot allocate memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, semantics, kernels and results as pa_decode_step, but the
 * workspace is a static device array of the library, PA_NOALLOC_SCRATCH_BYTES
 * (16 MiB) per GPU, which each GPU the library runs on holds until the
 * process ends; the plan crosses to the device through the pool's reserved
 * staging buffers.  The call makes no device or pinned-host allocation
 * (hipMalloc, hipHostMalloc, hipFree or a library routine that allocates);
 * host bookkeeping uses ordinary heap memory, and timing (pa_timing_enable)
 * creates its events when on.  The array used is that of the device
 * `stream` belongs to (the current device for NULL).
 * Every call on one GPU shares that GPU's array and leaves its contents
 * there: calls that may overlap on one GPU (different streams, or other
 * threads) race and must be ordered by the caller; successive calls on one
 * stream are ordered by the stream.
 * Errors: as pa_decode_step, checked before anything changes;
 *   PA_ERR_INVALID_ARG also when the step's workspace (pa_decode_step_
 *   workspace_bytes) exceeds PA_NOALLOC_SCRATCH_BYTES or its plan exceeds
 *   the pool's reserved staging buffers; PA_ERR_DEVICE if the array's
 *   address cannot be obtained. */
#define PA_NOALLOC_SCRATCH_BYTES (16u << 20)
pa_status pa_decode_step_noalloc(pa_pool* pool, const int64_t* seqs, int32_t B, int32_t num_heads,
                                 const void* k_new, const void* v_new, const void* q, void* out,
                                 int64_t* slots_out, void* stream);

/* Workspace bytes pa_verify_step needs for this batch (sized for the lengths
 * after its appends).  0 if the arguments are invalid. */
size_t pa_verify_step_workspace_bytes(const pa_pool* pool, const int64_t* seqs, const int32_t* q_lens,
                                      int32_t B, int32_t num_heads);

/* Multi-token step (speculative verification, short chunks): append
 * q_lens[b] >= 1 tokens to each sequence (pa_append_batch, all or nothing),
 * store their K/V rows and compute causal attention for those q_lens[b]
 * rows, the last positions of the sequence ([ferrum] paged_attention with
 * q_tokens = q_lens[b]: row t sees keys j <= L - q_lens[b] + t, L the length
 * after the append).  All q_lens[b] * G query columns of a sequence share
 * each K/V page load of the split-K decode kernels.
 * seqs: host [B], each at most once; q_lens: host [B]; R = sum q_lens;
 * k_new, v_new: device [R][num_kv_heads][head_dim]; q, out: device
 * [R][num_heads][head_dim] (rows sequence-major, as pa_prefill_chunk);
 * ws: at least pa_verify_step_workspace_bytes(...) bytes, 256-byte aligned;
 * slots_out: host [R] or NULL.
 * Needs bf16, int8 or E4M3 pages, head_dim 64 or 128, block_size 16 or 32 and
 * q_lens[b] * (num_heads / num_kv_heads) <= 32.
 * Errors: as pa_decode_step; PA_ERR_INVALID_ARG for a repeated sequence, a
 *   q_len < 1 or a shape the kernels do not cover, before anything changes. */
pa_status pa_verify_step(pa_pool* pool, const int64_t* seqs, const int32_t* q_lens, int32_t B,
                         int32_t num_heads, const void* k_new, const void* v_new, const void* q, void* out,
                         void* ws, size_t ws_bytes, int64_t* slots_out, void* stream);

/* Workspace bytes pa_prefill_chunk needs.  0 if the arguments are invalid. */
size_t pa_prefill_workspace_bytes(const pa_pool* pool, const int64_t* seqs,
                                  const int32_t* q_lens, int32_t B, int32_t num_heads);

/* Chunked causal prefill ([ferrum] paged_attention with q_tokens > 1): the
 * q_lens[b] query rows of sequence b are its LAST q_lens[b] positions, whose
 * K/V must already be appended and cached.  With L = length(seqs[b]), row t
 * (0 <= t < q_lens[b]) sees keys j <= L - q_lens[b] + t (bottom-right causal
 * mask, the same rule as [lecture19] CachedDecoder):
 *     out[r][h] = sum_{j visible} softmax(s)_j V_j[g],  r = row offset of b + t
 * seqs, q_lens: host [B]; q, out: device [sum q_lens][num_heads][head_dim];
 * ws: as for pa_decode.
 * Chunks whose every q_lens[b] * G <= 32 (on the MFMA decode shapes) run on
 * the split-K decode kernels; longer ones on the prefill kernel.
 * Errors: PA_ERR_UNKNOWN_SEQ, PA_ERR_INVALID_ARG (q_lens[b] < 1 or > L,
 *   head mismatch, small ws, NULL pointers), PA_ERR_DEVICE. */
pa_status pa_prefill_chunk(pa_pool* pool, const int64_t* seqs, const int32_t* q_lens,
                           int32_t B, int32_t num_heads, const void* q, void* out,
                           void* ws, size_t ws_bytes, void* stream);

/* ----------------------------------------------------------- inspection --- */
/* Synchronous host reads of the metadata ([PagedPool] sequence_length,
 * page_table, the per-block ref_count, the accounting properties and
 * validate).  They never touch the device. */
pa_status pa_seq_len(const pa_pool* pool, int64_t seq, int32_t* len);
/* out: host [cap]; *n receives the table length (only min(n, cap) written);
 * a page a window released reads -1. */
pa_status pa_block_table(const pa_pool* pool, int64_t seq, int32_t* out, int32_t cap, int32_t* n);
pa_status pa_refcount(const pa_pool* pool, int32_t block, int32_t* rc);
pa_status pa_stats(const pa_pool* pool, pa_pool_stats* stats);
/* [PagedPool] validate: refcount == table references + prefix-cache pins,
 * free <=> refcount 0, table length == ceil(len / block_size), no block
 * twice in one table, fill of a block some table holds in [1, block_size]
 * (a block only pins hold has fill 0 and is not free), logical >= payload.
 * Returns PA_ERR_INVALID_ARG with the broken invariant in pa_last_error. */
pa_status pa_validate(const pa_pool* pool);
/* Number of live sequences; ids_out (host [cap], may be NULL) receives them
 * in ascending order. */
pa_status pa_sequences(const pa_pool* pool, int64_t* ids_out, int32_t cap, int32_t* n);

/* The split-K work list a decode call (pa_decode, or with q_lens the verify
 * step and short prefill chunks) builds for this batch, in launch order;
 * host only, for tests and debugging (no page defines the partition: it is
 * this library's split of [ferrum] paged_attention's key loop, merged by
 * [lecture19] online_softmax_stats).  q_lens NULL = one row per sequence.
 * *pages_per_range: the pages of one range; items: host [cap_items][16]
 * ints per work item: batch row b, range c (compact pages [c * pages_per_range,
 * min(visited, (c + 1) * pages_per_range)) of the sequence's visited pages),
 * length L, first query row, q_len, sinks, recent (2^29 without a window),
 * sink pages, gap, table offset, first split-K partial row-head (-1: the
 * sequence is one range), 0, then the block of compact page
 * c * pages_per_range + w for waves w < 4 (0 past the range); tables: host
 * [cap_tables], the visited pages of every row from its table offset:
 * compact page i is page i for i < sink pages, else page i + gap.
 * *n_items / *n_tables receive the counts; only what fits is written.
 * Errors: as the plan of pa_decode (PA_ERR_UNKNOWN_SEQ, PA_ERR_INVALID_ARG
 * for an empty sequence, q_lens[b] outside 1..length, a head mismatch or
 * NULL outputs). */
pa_status pa_decode_work_items(const pa_pool* pool, const int64_t* seqs, const int32_t* q_lens, int32_t B,
                               int32_t num_heads, int32_t* pages_per_range, int32_t* items, int32_t cap_items,
                               int32_t* n_items, int32_t* tables, int64_t cap_tables, int64_t* n_tables);
/* Message of the last failed call on this thread ("" if none). */
const char* pa_last_error(void);

/* ---------------------------------------------------------------- timing --- */
/* Kernel timing with HIP events that each timed kernel's dispatch carries
 * on the stream it is launched on (hipExtLaunchKernel: the events take the
 * kernel's start and end; nothing else is put on the stream).  Off by
 * default.  pa_timing_read synchronizes on the events and returns the summed
 * duration and launch count of one kernel family since the last reset. */
typedef enum {
  PA_KERNEL_DECODE = 0,   /* decode partial (split-K) kernel */
  PA_KERNEL_MERGE = 1,    /* log-sum-exp merge */
  PA_KERNEL_PREFILL = 2,  /* chunked prefill */
  PA_KERNEL_CACHE = 3,    /* reshape_and_cache */
  PA_KERNEL_COPY = 4,     /* copy-on-write block copies */
  PA_KERNEL_COUNT = 5
} pa_kernel;
pa_status pa_timing_enable(int on);
/* Which kernel families get events while timing is on: bit k = pa_kernel k
 * (default all).  A timed launch still spaces the stream's kernels by a few
 * microseconds, so a caller timing whole steps can time only the family it
 * reports (and only some of the steps). */
pa_status pa_timing_select(uint32_t kernel_mask);
pa_status pa_timing_reset(void);
pa_status pa_timing_read(int32_t kernel, double* total_ms, int64_t* launches);
/* Per-launch durations (ms, launch order) of one kernel family since the
 * last reset: the first min(cap, *n) go to ms_out (host [cap], may be NULL
 * when cap is 0); *n receives the count.  Synchronizes like pa_timing_read.
 * Errors: PA_ERR_INVALID_ARG for a bad kernel id, a negative cap, a NULL n
 * or a NULL ms_out with cap > 0. */
pa_status pa_timing_samples(int32_t kernel, float* ms_out, int64_t cap, int64_t* n);

#ifdef __cplusplus
}
#endif
#endif /* PAGEDATTN_H */
