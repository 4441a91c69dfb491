// Device work plans for decode and prefill: which (sequence, KV head, page
// range) each workgroup handles, where the block tables and split-K partial
// results live inside the caller's workspace, and the kernel argument blocks.
//
// Host-only (no HIP types) so it builds and is checked on a CPU machine.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "pool.hpp"

namespace pa {

constexpr size_t kWsAlign = 256;
constexpr int32_t kNoWindowRecent = 1 << 29;  // "recent" of a sequence without a window
constexpr int kDecodeWaves = 4;  // waves per decode workgroup
constexpr int kWorkInts = 16;    // ints per decode work item

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Geometry of a pool.  dtype: 0 = fp32, 1 = bf16, 2 = int8 codes, 3 = E4M3
// codes; 8-bit codes come with one fp32 scale per (token, KV head) row (q /
// out / new rows are then bf16).
struct PoolGeom {
  int32_t num_blocks, block_size, num_kv_heads, head_dim, dtype;
  bool q8() const { return dtype == 2 || dtype == 3; }  // 8-bit codes + fp32 row scales
  bool fp8() const { return dtype == 3; }               // the codes are E4M3 floats
  // Element size of q, out, k_new and v_new.
  int32_t io_elt() const { return dtype == 0 ? 4 : 2; }
  size_t page_elems() const { return static_cast<size_t>(block_size) * head_dim; }
  // Bytes of one (block, KV head) page: codes then scales for 8-bit pools.
  size_t page_bytes() const {
    if (q8()) return page_elems() + 4 * static_cast<size_t>(block_size);
    return page_elems() * (dtype == 1 ? 2 : 4);
  }
  size_t block_bytes() const { return static_cast<size_t>(num_kv_heads) * page_bytes(); }
};


// Kernel arguments of the decode partial kernels.  Every pointer is device
// memory inside the workspace, except q / out / pools.  Sequence b has
// q_len_b = q_start[b+1] - q_start[b] query rows (its last q_len_b
// positions; 1 for plain decode); a split sequence keeps one partial row per
// (partition, query row, head).
struct DecodeArgs {
  const void* k_pool;
  const void* v_pool;
  const void* q;            // [R][Hq][D], R = q_start[B]
  void* out;                // [R][Hq][D]
  const int32_t* ctx_len;   // [B] tokens per sequence
  const int32_t* tbl_off;   // [B] offset of the sequence's table in `tables`
  const int32_t* tables;    // concatenated block tables of the visited pages, by compact
                            // page index (see seq_win)
  const int32_t* q_start;   // [B+1] first query row of b
  const int32_t* work;      // [n_work][kWorkInts]: b, partition c, L, row0, q_len, sinks,
                            // recent, sink pages, gap, table offset, part_base, 0, then the
                            // block of compact page c * pages_per_part + w for waves w < 4
                            // (everything a workgroup needs before its first page, in one
                            // 64-byte scalar load)
  const int32_t* part_base; // [B] first partial row-head of b, or -1 = single partition;
                            // row-head of (partition c, row t, head h) =
                            // part_base + (c * q_len_b + t) * Hq + h
  float* part_m;            // [row-heads]
  float* part_l;            // [row-heads]
  float* part_acc;          // [row-heads][D]
  const int32_t* merge_rows;// [n_merge][4] per query row of a split sequence: its output
                            // row, the partial row-head of its head 0 in partition 0,
                            // the row-head stride between partitions, the partitions
  const int32_t* seq_win;   // [B][4] = (sinks, recent, sink pages, gap): the pages
                            // visited are the compact indices i < n_visit = nblk - gap,
                            // page i for i < sink pages, else page i + gap; a key p is
                            // visible to a row whose causal limit is lim (p < lim) if
                            // p < sinks or p >= lim - recent (no window: recent huge)
  const int32_t* n_parts_of;// [B] partitions of b
  int32_t batch, num_heads, num_kv_heads, group;
  int32_t pages_per_part;
  int32_t n_work, n_merge;
  int32_t max_cols;         // max over b of q_len_b * group (MFMA columns)
  float scale_log2;         // log2(e) / sqrt(head_dim)
};

struct DecodePlan {
  std::vector<int32_t> meta;  // host image of the metadata region
  size_t meta_bytes = 0;      // aligned
  size_t part_m_off = 0, part_l_off = 0, part_acc_off = 0, total_bytes = 0;
  size_t ctx_off = 0, tbl_off_off = 0, tables_off = 0, qstart_off = 0, work_off = 0, base_off = 0,
         merge_off = 0, nparts_off = 0, win_off = 0, slots_off = 0;  // byte offsets in the workspace
  int32_t n_work = 0, n_merge = 0, n_parts = 0, pages_per_part = 0, batch = 0;
  int32_t n_rows = 0, max_q_len = 1;
  int64_t total_pages = 0;
};

// Build the decode plan for `seqs`.  Validates the batch (known sequences,
// non-empty contexts, 1 <= q_lens[b] <= length); returns kUnknownSeq /
// kInvalidArg with msg.
// `tokens_per_part` = 0 chooses the partition size automatically.
// `extra_tokens` (nullable, [B]) sizes the plan as if row b had that many
// more tokens: such a plan is for sizing only (its offsets and sizes are
// set, its `meta` is left empty).  `q_lens` (nullable = all 1) gives the query rows of
// each sequence.  `slot_count` reserves an int64 slot array (slots_off) for
// the caller to fill.
Status build_decode_plan(const BlockPool& pool, const int64_t* seqs, int32_t B, int32_t num_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t tokens_per_part,
                         const int32_t* extra_tokens, const int32_t* q_lens, int32_t slot_count,
                         DecodePlan* plan, std::string* msg);

// Kernel arguments of the prefill kernels.
struct PrefillArgs {
  const void* k_pool;
  const void* v_pool;
  const void* q;            // [R][Hq][D], R = sum q_lens
  void* out;                // [R][Hq][D]
  const int32_t* ctx_len;   // [B]
  const int32_t* tbl_off;   // [B]
  const int32_t* tables;
  const int32_t* q_start;   // [B+1] first row of b
  const int32_t* tiles;     // [n_tiles][2] = (b, first query row of the tile within b)
  const int32_t* row_seq;   // [R] sequence of each row (generic kernel)
  const int32_t* seq_win;   // [B][4] as in DecodeArgs (sinks, recent; no window: 0, kNoWindowRecent)
  const void* zeros;        // 64 zero bytes (source of staged slots past a sequence's end)
  int32_t num_heads, num_kv_heads, group;
  int32_t n_tiles, n_rows;
  float scale_log2;
};

struct PrefillPlan {
  std::vector<int32_t> meta;
  size_t meta_bytes = 0, total_bytes = 0;
  size_t ctx_off = 0, tbl_off_off = 0, tables_off = 0, qstart_off = 0, tiles_off = 0,
         rowseq_off = 0, zeros_off = 0, win_off = 0;
  int32_t n_tiles = 0, n_rows = 0, batch = 0;
};

// `rows_per_tile` query rows (of one sequence) per prefill workgroup.
Status build_prefill_plan(const BlockPool& pool, const int64_t* seqs, const int32_t* q_lens,
                          int32_t B, int32_t num_heads, int32_t num_kv_heads, int32_t rows_per_tile,
                          PrefillPlan* plan, std::string* msg);

}  // namespace pa
