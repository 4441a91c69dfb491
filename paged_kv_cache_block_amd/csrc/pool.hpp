// Host-side bookkeeping of the paged KV pool: allocation order, refcounts,
// per-sequence block tables and lengths, preflighted append with
// copy-on-write, share / fork / release, accounting and invariants.
//
// Semantics follow abhik.ai "examples/pagedattention.py" (class KVPool:
// first free block in the authored allocation order, whole-block copy of a
// shared partial tail, fork, release) and the "Модуль 10" notebook's
// PagedKVPool (multi-token append preflight, share_prefix, fill / payload /
// waste / savings accounting, validate).  This translation unit has no HIP
// dependency so that it builds and is exercised on a CPU-only machine.
#pragma once

#include <cstdint>
#include <functional>
#include <queue>
#include <string>
#include <unordered_map>
#include <utility>
#include <vector>

namespace pa {

enum Status : int {
  kOk = 0,
  kInvalidArg = -1,
  kUnknownSeq = -2,
  kSeqExists = -3,
  kOutOfBlocks = -4,
  kDevice = -5,
};

constexpr int32_t kHole = -1;  // table entry of a page the window released

struct Sequence {
  int64_t length = 0;
  std::vector<int32_t> table;
  // Window (vladkulikov.com notebook "Модуль 10", streaming_keep_indices
  // with budget sinks + recent); sinks < 0: no window.
  int32_t sinks = -1, recent = 0;
  bool windowed() const { return sinks >= 0; }
  // Incremental window bookkeeping: the pages from the sink pages up to
  // scan_from are all released (the next release resumes there), and
  // hole_end is one past the last released page (0 if none).
  int64_t scan_from = 0;
  int64_t hole_end = 0;
};

struct PoolStats {
  int64_t allocated_blocks, free_blocks, physical_capacity_tokens, physical_payload_tokens,
      logical_tokens, internal_waste_tokens, sharing_savings_tokens;
};

class BlockPool {
 public:
  // `order` empty = identity.  Returns kInvalidArg (with msg) on bad input.
  static Status make(int32_t num_blocks, int32_t block_size, const int32_t* order,
                     BlockPool* out, std::string* msg);

  Status create(int64_t seq, std::string* msg);
  Status append(int64_t seq, int32_t n, int64_t* slots_out, std::string* msg);
  // append(seqs[i], n[i]) for i = 0..count-1 in order, slots concatenated in
  // slots_out.  All or nothing: on any failure every earlier append of the
  // batch is undone and the pool is exactly as before the call.
  Status append_batch(const int64_t* seqs, const int32_t* n, int32_t count, int64_t* slots_out,
                      std::string* msg);
  Status share(int64_t src, int64_t dst, int32_t prefix, std::string* msg);
  Status fork(int64_t src, int64_t dst, std::string* msg);
  Status release(int64_t seq, std::string* msg);
  // New sequence `seq` whose table is blocks[0..n_blocks) (each refcount + 1)
  // and whose length is `length`; ceil(length / block_size) must equal
  // n_blocks, the blocks must be live and distinct.
  Status adopt(int64_t seq, const int32_t* blocks, int32_t n_blocks, int64_t length, std::string* msg);
  // A reference held outside every table (the prefix cache's); only a live
  // block can be pinned.  unpin drops it (the block is freed at refcount 0).
  Status pin(int32_t block, std::string* msg);
  Status unpin(int32_t block, std::string* msg);
  int32_t pins(int32_t block) const { return pins_[block]; }
  // Give `seq` a (sinks, recent) window: each append then releases the
  // pages lying wholly between the sink pages and the window of its first
  // appended row (position p sees [p + 1 - recent, p]); their table entries
  // become kHole.
  Status set_window(int64_t seq, int32_t sinks, int32_t recent, std::string* msg);
  // Drop positions [new_length, length) (a rollback).  new_length may not
  // fall before evicted_end(seq): evicted positions cannot come back.
  Status truncate(int64_t seq, int64_t new_length, std::string* msg);
  // First position after the last released page (0 if none).
  int64_t evicted_end(const Sequence& s) const;

  const Sequence* find(int64_t seq) const;
  int32_t refcount(int32_t block) const { return refs_[block]; }
  int32_t num_blocks() const { return num_blocks_; }
  int32_t block_size() const { return block_size_; }
  int64_t free_count() const { return n_free_; }
  PoolStats stats() const;
  Status validate(std::string* msg) const;
  std::vector<int64_t> sequence_ids() const;

  // Blocks needed to append n tokens to `s` (the preflight count).
  int64_t blocks_needed(const Sequence& s, int64_t n) const;

  // Copy-on-write copies recorded since the last take_pending_copies().
  const std::vector<std::pair<int32_t, int32_t>>& pending_copies() const { return pending_; }
  std::vector<std::pair<int32_t, int32_t>> take_pending_copies();

  // Incremented by every mutation; lets callers cache derived device state.
  uint64_t version() const { return version_; }

 private:
  // First-touch values of every block an append_batch changed.
  struct UndoLog {
    std::unordered_map<int32_t, std::pair<int32_t, char>> blocks;  // block -> (refs, free)
  };

  void touch(int32_t block);
  int32_t allocate();
  void drop_ref(int32_t block);
  void evict(Sequence& s, int64_t first_new);
  std::vector<int32_t> fills() const;

  int32_t num_blocks_ = 0;
  int32_t block_size_ = 0;
  std::vector<int32_t> order_;  // rank -> block
  std::vector<int32_t> rank_;   // block -> rank
  std::vector<int32_t> refs_;
  std::vector<int32_t> pins_;   // references held outside the tables
  std::vector<char> is_free_;
  int64_t n_free_ = 0;
  // Ranks of free blocks, smallest first; entries of blocks allocated since
  // they were pushed are stale and skipped (an undone batch re-pushes).
  std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>> free_heap_;
  std::unordered_map<int64_t, Sequence> seqs_;
  std::vector<std::pair<int32_t, int32_t>> pending_;
  uint64_t version_ = 0;
  UndoLog* undo_ = nullptr;  // set while append_batch runs
};

}  // namespace pa
