// Host bookkeeping of the paged KV pool.  See pool.hpp for the sources.
#include "pool.hpp"

#include <algorithm>
#include <string>

namespace pa {

namespace {
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
}  // namespace

Status BlockPool::make(int32_t num_blocks, int32_t block_size, const int32_t* order,
                       BlockPool* out, std::string* msg) {
  if (num_blocks <= 0 || block_size <= 0) {
    *msg = "num_blocks and block_size must be positive";
    return kInvalidArg;
  }
  BlockPool p;
  p.num_blocks_ = num_blocks;
  p.block_size_ = block_size;
  p.order_.resize(num_blocks);
  p.rank_.assign(num_blocks, -1);
  for (int32_t r = 0; r < num_blocks; ++r) {
    int32_t b = order ? order[r] : r;
    if (b < 0 || b >= num_blocks || p.rank_[b] != -1) {
      *msg = "allocation_order must be a full permutation of 0..num_blocks-1";
      return kInvalidArg;
    }
    p.order_[r] = b;
    p.rank_[b] = r;
  }
  p.refs_.assign(num_blocks, 0);
  p.pins_.assign(num_blocks, 0);
  p.is_free_.assign(num_blocks, 1);
  p.n_free_ = num_blocks;
  std::vector<int32_t> ranks(num_blocks);
  for (int32_t r = 0; r < num_blocks; ++r) ranks[r] = r;
  p.free_heap_ = decltype(p.free_heap_)(std::greater<int32_t>(), std::move(ranks));
  *out = std::move(p);
  return kOk;
}

const Sequence* BlockPool::find(int64_t seq) const {
  auto it = seqs_.find(seq);
  return it == seqs_.end() ? nullptr : &it->second;
}

void BlockPool::touch(int32_t block) {
  if (undo_) undo_->blocks.emplace(block, std::make_pair(refs_[block], is_free_[block]));
}

int32_t BlockPool::allocate() {
  // Caller has preflighted: a free block exists.
  int32_t block;
  do {
    block = order_[free_heap_.top()];
    free_heap_.pop();
  } while (!is_free_[block]);
  touch(block);
  is_free_[block] = 0;
  --n_free_;
  refs_[block] = 1;
  return block;
}

void BlockPool::drop_ref(int32_t block) {
  touch(block);
  if (--refs_[block] == 0) {
    is_free_[block] = 1;
    ++n_free_;
    free_heap_.push(rank_[block]);
  }
}

void BlockPool::evict(Sequence& s, int64_t first_new) {
  const int64_t sink_pages = ceil_div(s.sinks, block_size_);
  const int64_t lo = first_new + 1 - s.recent;
  const int64_t end = std::min(std::max<int64_t>(lo, 0) / block_size_, first_new / block_size_);
  // Pages below scan_from are released already: each page is visited once
  // over the sequence's appends instead of on every append.
  for (int64_t j = std::max(sink_pages, s.scan_from); j < end; ++j) {
    if (s.table[j] == kHole) continue;
    drop_ref(s.table[j]);
    s.table[j] = kHole;
    s.hole_end = std::max(s.hole_end, j + 1);
  }
  s.scan_from = std::max(s.scan_from, end);
}

int64_t BlockPool::evicted_end(const Sequence& s) const { return s.hole_end * block_size_; }

Status BlockPool::set_window(int64_t seq, int32_t sinks, int32_t recent, std::string* msg) {
  auto it = seqs_.find(seq);
  if (it == seqs_.end()) {
    *msg = "unknown sequence: " + std::to_string(seq);
    return kUnknownSeq;
  }
  if (sinks < 0 || recent < 0 || static_cast<int64_t>(sinks) + recent < 1 ||
      static_cast<int64_t>(sinks) + recent > INT32_MAX / 2) {
    *msg = "sinks and recent must be >= 0 with 1 <= sinks + recent";
    return kInvalidArg;
  }
  it->second.sinks = sinks;
  it->second.recent = recent;
  it->second.scan_from = 0;  // other sink pages: the next release scans from them
  ++version_;
  return kOk;
}

Status BlockPool::truncate(int64_t seq, int64_t new_length, std::string* msg) {
  auto it = seqs_.find(seq);
  if (it == seqs_.end()) {
    *msg = "unknown sequence: " + std::to_string(seq);
    return kUnknownSeq;
  }
  Sequence& s = it->second;
  if (new_length < 0 || new_length > s.length) {
    *msg = "new_length must be in 0..length(seq)";
    return kInvalidArg;
  }
  if (new_length < evicted_end(s)) {
    *msg = "rollback lies outside the retained interval (evicted positions cannot come back)";
    return kInvalidArg;
  }
  const size_t keep = static_cast<size_t>(ceil_div(new_length, block_size_));
  for (size_t j = keep; j < s.table.size(); ++j)
    if (s.table[j] != kHole) drop_ref(s.table[j]);
  s.table.resize(keep);
  s.length = new_length;
  s.scan_from = std::min<int64_t>(s.scan_from, static_cast<int64_t>(keep));
  ++version_;
  return kOk;
}

Status BlockPool::create(int64_t seq, std::string* msg) {
  if (seqs_.count(seq)) {
    *msg = "sequence already exists: " + std::to_string(seq);
    return kSeqExists;
  }
  seqs_.emplace(seq, Sequence{});
  ++version_;
  return kOk;
}

int64_t BlockPool::blocks_needed(const Sequence& s, int64_t n) const {
  if (n == 0) return 0;
  int64_t need = 0, room = 0;
  int64_t remainder = s.length % block_size_;
  if (remainder) {
    if (refs_[s.table.back()] > 1) need += 1;  // copy of the shared partial tail
    room = block_size_ - remainder;
  }
  need += ceil_div(std::max<int64_t>(0, n - room), block_size_);
  return need;
}

Status BlockPool::append(int64_t seq, int32_t n, int64_t* slots_out, std::string* msg) {
  auto it = seqs_.find(seq);
  if (it == seqs_.end()) {
    *msg = "unknown sequence: " + std::to_string(seq);
    return kUnknownSeq;
  }
  if (n < 0 || (n > 0 && !slots_out)) {
    *msg = "n_tokens must be >= 0 and slots_out non-NULL when n_tokens > 0";
    return kInvalidArg;
  }
  Sequence& s = it->second;
  int64_t need = blocks_needed(s, n);
  if (need > free_count()) {
    *msg = "need " + std::to_string(need) + " free blocks, " + std::to_string(free_count()) +
           " remain";
    return kOutOfBlocks;
  }
  if (n == 0) return kOk;
  if (s.length % block_size_) {
    int32_t old = s.table.back();
    if (refs_[old] > 1) {
      int32_t fresh = allocate();
      pending_.emplace_back(old, fresh);
      s.table.back() = fresh;
      drop_ref(old);  // old stays referenced by another sequence
    }
  }
  int64_t first = s.length;
  int64_t total = s.length + n;
  while (static_cast<int64_t>(s.table.size()) < ceil_div(total, block_size_))
    s.table.push_back(allocate());
  s.length = total;
  for (int64_t p = first; p < total; ++p)
    slots_out[p - first] =
        static_cast<int64_t>(s.table[p / block_size_]) * block_size_ + p % block_size_;
  if (s.windowed()) evict(s, first);
  ++version_;
  return kOk;
}

Status BlockPool::append_batch(const int64_t* seqs, const int32_t* n, int32_t count,
                               int64_t* slots_out, std::string* msg) {
  if (count < 0 || (count > 0 && (!seqs || !n))) {
    *msg = "count must be >= 0 with non-NULL seqs and n_tokens";
    return kInvalidArg;
  }
  // Fast path: distinct, known sequences whose appends together need no more
  // blocks than are free (each need taken on the state before the batch; an
  // earlier append can only lower a later one's need, by dropping a shared
  // tail's reference or releasing pages behind a window) cannot fail, so
  // they run without an undo log.
  if (count > 0) {
    std::vector<int64_t> ids(seqs, seqs + count);
    std::sort(ids.begin(), ids.end());
    bool fast = std::adjacent_find(ids.begin(), ids.end()) == ids.end();
    int64_t need = 0;
    for (int32_t i = 0; fast && i < count; ++i) {
      auto it = seqs_.find(seqs[i]);
      fast = it != seqs_.end() && n[i] >= 0 && (n[i] == 0 || slots_out);
      if (fast) need += blocks_needed(it->second, n[i]);
    }
    if (fast && need <= free_count()) {
      int64_t offset = 0;
      for (int32_t i = 0; i < count; ++i) {
        const Status st = append(seqs[i], n[i], slots_out ? slots_out + offset : nullptr, msg);
        if (st != kOk) return st;  // unreachable: checked above
        offset += n[i];
      }
      return kOk;
    }
  }
  // Undo log: the first-seen state of every touched sequence and of every
  // block whose refcount or free flag the batch changed (allocations,
  // copy-on-write drops, window releases), and the pending-copy list
  // length.  Restoring the free flags restores the free set, and with it
  // the allocation order (stale heap entries are skipped).
  std::unordered_map<int64_t, Sequence> saved;
  UndoLog log;
  const size_t pending_before = pending_.size();
  const uint64_t version_before = version_;
  undo_ = &log;
  int64_t offset = 0;
  Status s = kOk;
  int32_t i = 0;
  for (; i < count; ++i) {
    if (n[i] > 0 && !slots_out) {
      *msg = "slots_out must be non-NULL when tokens are appended";
      s = kInvalidArg;
      break;
    }
    auto it = seqs_.find(seqs[i]);
    if (it != seqs_.end() && !saved.count(seqs[i])) saved.emplace(seqs[i], it->second);
    s = append(seqs[i], n[i], slots_out ? slots_out + offset : nullptr, msg);
    if (s != kOk) break;
    offset += n[i];
  }
  undo_ = nullptr;
  if (s == kOk) return kOk;
  for (auto& kv : saved) seqs_[kv.first] = std::move(kv.second);
  for (const auto& kv : log.blocks) {
    const int32_t b = kv.first;
    refs_[b] = kv.second.first;
    const char was_free = kv.second.second;
    if (is_free_[b] != was_free) {
      is_free_[b] = was_free;
      n_free_ += was_free ? 1 : -1;
      if (was_free) free_heap_.push(rank_[b]);
    }
  }
  pending_.resize(pending_before);
  version_ = version_before;
  *msg = "append_batch entry " + std::to_string(i) + ": " + *msg;
  return s;
}

Status BlockPool::share(int64_t src, int64_t dst, int32_t prefix, std::string* msg) {
  auto it = seqs_.find(src);
  if (it == seqs_.end()) {
    *msg = "unknown sequence: " + std::to_string(src);
    return kUnknownSeq;
  }
  if (prefix < 0 || prefix > it->second.length) {
    *msg = "prefix_tokens must be in 0..length(src)";
    return kInvalidArg;
  }
  if (prefix < evicted_end(it->second)) {
    *msg = "prefix_tokens ends among positions a window released";
    return kInvalidArg;
  }
  if (seqs_.count(dst)) {
    *msg = "sequence already exists: " + std::to_string(dst);
    return kSeqExists;
  }
  Sequence child;
  child.length = prefix;
  child.table.assign(it->second.table.begin(),
                     it->second.table.begin() + ceil_div(prefix, block_size_));
  child.sinks = it->second.sinks;
  child.recent = it->second.recent;
  child.hole_end = it->second.hole_end;  // <= the copied pages: prefix >= evicted_end(src)
  child.scan_from = std::min<int64_t>(it->second.scan_from, static_cast<int64_t>(child.table.size()));
  for (int32_t b : child.table)
    if (b != kHole) ++refs_[b];
  seqs_.emplace(dst, std::move(child));
  ++version_;
  return kOk;
}

Status BlockPool::fork(int64_t src, int64_t dst, std::string* msg) {
  const Sequence* s = find(src);
  if (!s) {
    *msg = "unknown sequence: " + std::to_string(src);
    return kUnknownSeq;
  }
  return share(src, dst, static_cast<int32_t>(s->length), msg);
}

Status BlockPool::release(int64_t seq, std::string* msg) {
  auto it = seqs_.find(seq);
  if (it == seqs_.end()) {
    *msg = "unknown or released sequence: " + std::to_string(seq);
    return kUnknownSeq;
  }
  for (int32_t b : it->second.table)
    if (b != kHole) drop_ref(b);
  seqs_.erase(it);
  ++version_;
  return kOk;
}

Status BlockPool::adopt(int64_t seq, const int32_t* blocks, int32_t n_blocks, int64_t length,
                        std::string* msg) {
  if (seqs_.count(seq)) {
    *msg = "sequence already exists: " + std::to_string(seq);
    return kSeqExists;
  }
  if (n_blocks < 0 || length < 0 || (n_blocks > 0 && !blocks) || ceil_div(length, block_size_) != n_blocks) {
    *msg = "adopted blocks must cover the length exactly";
    return kInvalidArg;
  }
  std::vector<int32_t> table(blocks, blocks + n_blocks);
  std::vector<int32_t> sorted = table;
  std::sort(sorted.begin(), sorted.end());
  if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end()) {
    *msg = "adopted blocks must be distinct";
    return kInvalidArg;
  }
  for (int32_t b : table)
    if (b < 0 || b >= num_blocks_ || refs_[b] == 0) {
      *msg = "adopted blocks must be live";
      return kInvalidArg;
    }
  for (int32_t b : table) ++refs_[b];
  Sequence s;
  s.length = length;
  s.table = std::move(table);
  seqs_.emplace(seq, std::move(s));
  ++version_;
  return kOk;
}

Status BlockPool::pin(int32_t block, std::string* msg) {
  if (block < 0 || block >= num_blocks_ || refs_[block] == 0) {
    *msg = "only a live block can be pinned";
    return kInvalidArg;
  }
  ++refs_[block];
  ++pins_[block];
  ++version_;
  return kOk;
}

Status BlockPool::unpin(int32_t block, std::string* msg) {
  if (block < 0 || block >= num_blocks_ || pins_[block] == 0) {
    *msg = "block is not pinned";
    return kInvalidArg;
  }
  --pins_[block];
  drop_ref(block);
  ++version_;
  return kOk;
}

std::vector<std::pair<int32_t, int32_t>> BlockPool::take_pending_copies() {
  std::vector<std::pair<int32_t, int32_t>> out;
  out.swap(pending_);
  return out;
}

std::vector<int32_t> BlockPool::fills() const {
  std::vector<int32_t> fill(num_blocks_, 0);
  for (const auto& kv : seqs_) {
    const Sequence& s = kv.second;
    for (size_t j = 0; j < s.table.size(); ++j) {
      if (s.table[j] == kHole) continue;
      int64_t used = std::min<int64_t>(block_size_, s.length - static_cast<int64_t>(j) * block_size_);
      fill[s.table[j]] = std::max<int32_t>(fill[s.table[j]], static_cast<int32_t>(used));
    }
  }
  return fill;
}

PoolStats BlockPool::stats() const {
  PoolStats st{};
  st.free_blocks = free_count();
  st.allocated_blocks = num_blocks_ - st.free_blocks;
  st.physical_capacity_tokens = st.allocated_blocks * block_size_;
  std::vector<int32_t> fill = fills();
  int64_t payload = 0;
  for (int32_t b = 0; b < num_blocks_; ++b)
    if (refs_[b]) payload += fill[b];
  int64_t logical = 0;
  for (const auto& kv : seqs_) logical += kv.second.length;
  st.physical_payload_tokens = payload;
  st.logical_tokens = logical;
  st.internal_waste_tokens = st.physical_capacity_tokens - payload;
  st.sharing_savings_tokens = logical - payload;
  return st;
}

// The invariants the [PagedPool] validate method states, recomputed from the
// tables: (1) a table holds ceil(length / block_size) pages, no block twice,
// and never a released partial tail; (2) a block's refcount is the number of
// tables that list it plus its pins; (3) a block is free exactly when its
// refcount is 0, and every free block can be drawn from the free heap; (4) a
// block's fill is 0 unless a table lists it, then 1..block_size; (5) the
// logical tokens are at least the physical payload.
Status BlockPool::validate(std::string* msg) const {
  auto broken = [msg](const std::string& what, int64_t at) {
    *msg = "pool invariant broken: " + what + " (at " + std::to_string(at) + ")";
    return kInvalidArg;
  };
  std::vector<int32_t> listed_by(num_blocks_, 0);
  std::vector<int64_t> stamp(num_blocks_, -1);  // last table (by visit number) that listed the block
  int64_t visit = 0;
  for (const auto& kv : seqs_) {
    const Sequence& s = kv.second;
    if (s.length < 0 || static_cast<int64_t>(s.table.size()) != ceil_div(s.length, block_size_))
      return broken("table size is not ceil(length / block_size) for sequence", kv.first);
    const size_t n = s.table.size();
    int64_t last_hole = 0;
    for (size_t i = 0; i < n; ++i) {
      const int32_t b = s.table[i];
      if (b == kHole) {
        if (i + 1 == n && s.length % block_size_)
          return broken("the partially filled last page is released in sequence", kv.first);
        last_hole = static_cast<int64_t>(i) + 1;
        continue;
      }
      if (b < 0 || b >= num_blocks_) return broken("block id outside the pool in sequence", kv.first);
      if (stamp[b] == visit) return broken("a block appears twice in the table of sequence", kv.first);
      stamp[b] = visit;
      ++listed_by[b];
    }
    if (last_hole != s.hole_end)
      return broken("recorded end of the released pages is stale in sequence", kv.first);
    if (s.windowed()) {
      const int64_t sink_pages = ceil_div(s.sinks, block_size_);
      for (int64_t j = sink_pages; j < std::min<int64_t>(s.scan_from, static_cast<int64_t>(n)); ++j)
        if (s.table[j] != kHole) return broken("a page below the release cursor is resident in sequence", kv.first);
    }
    ++visit;
  }
  std::vector<char> drawable(num_blocks_, 0);
  for (auto heap = free_heap_; !heap.empty(); heap.pop()) {
    const int32_t r = heap.top();
    if (r < 0 || r >= num_blocks_) return broken("free-heap rank outside the pool", r);
    drawable[order_[r]] = 1;
  }
  const std::vector<int32_t> fill = fills();
  int64_t free_blocks = 0;
  for (int32_t b = 0; b < num_blocks_; ++b) {
    if (refs_[b] != listed_by[b] + pins_[b]) return broken("refcount != table references + pins of block", b);
    const bool is_free = is_free_[b] != 0;
    if (is_free != (refs_[b] == 0)) return broken("free flag disagrees with the refcount of block", b);
    if (is_free && !drawable[b]) return broken("free block missing from the free heap", b);
    free_blocks += is_free;
    const int32_t lo = listed_by[b] ? 1 : 0, hi = listed_by[b] ? block_size_ : 0;
    if (fill[b] < lo || fill[b] > hi) return broken("fill outside its range for block", b);
  }
  if (free_blocks != n_free_) return broken("free-block counter differs from the free flags", n_free_);
  const PoolStats st = stats();
  if (st.logical_tokens < st.physical_payload_tokens)
    return broken("physical payload tokens exceed logical tokens", st.physical_payload_tokens);
  return kOk;
}

std::vector<int64_t> BlockPool::sequence_ids() const {
  std::vector<int64_t> ids;
  ids.reserve(seqs_.size());
  for (const auto& kv : seqs_) ids.push_back(kv.first);
  std::sort(ids.begin(), ids.end());
  return ids;
}

}  // namespace pa
