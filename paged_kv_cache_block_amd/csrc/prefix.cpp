// Prefix-hash block reuse.  See prefix.hpp.
#include "prefix.hpp"

namespace pa {

size_t PrefixCache::EdgeHash::operator()(const Edge& e) const {
  // 64-bit FNV-1a over the parent id and the token ids.
  uint64_t h = 1469598103934665603ull;
  auto mix = [&h](uint64_t v) {
    for (int i = 0; i < 8; ++i) {
      h ^= (v >> (8 * i)) & 0xff;
      h *= 1099511628211ull;
    }
  };
  mix(static_cast<uint64_t>(e.parent));
  for (int32_t t : e.tokens) mix(static_cast<uint32_t>(t));
  return static_cast<size_t>(h);
}

std::string PrefixCache::root_key(const std::string& scope, const std::string& revision) {
  // Length-prefixed so that no two (scope, revision) pairs share a key.
  return std::to_string(scope.size()) + ":" + scope + revision;
}

int64_t PrefixCache::walk(const std::string& scope, const std::string& revision, const int32_t* tokens,
                          int64_t n, int32_t block_size, std::vector<int64_t>* path) const {
  auto r = roots_.find(root_key(scope, revision));
  if (r == roots_.end()) return 0;
  int64_t parent = -(r->second + 1);
  int64_t hit = 0;
  Edge probe;
  for (int64_t end = block_size; end <= n; end += block_size) {
    probe.parent = parent;
    probe.tokens.assign(tokens + end - block_size, tokens + end);
    auto it = edges_.find(probe);
    if (it == edges_.end()) break;
    parent = it->second;
    if (path) path->push_back(parent);
    hit = end;
  }
  return hit;
}

int64_t PrefixCache::lookup(const std::string& scope, const std::string& revision, const int32_t* tokens,
                            int64_t n) const {
  if (block_size_ == 0 || n <= 0) return 0;
  return walk(scope, revision, tokens, n, block_size_, nullptr);
}

Status PrefixCache::attach(BlockPool& pool, int64_t seq, const std::string& scope,
                           const std::string& revision, const int32_t* tokens, int64_t n, int64_t* hit,
                           std::string* msg) {
  if (n < 0 || (n > 0 && !tokens)) {
    *msg = "n_tokens must be >= 0 with non-NULL tokens";
    return kInvalidArg;
  }
  std::vector<int64_t> path;
  int64_t h = 0;
  if (block_size_ != 0 && n > 0) h = walk(scope, revision, tokens, n, block_size_, &path);
  std::vector<int32_t> blocks;
  blocks.reserve(path.size());
  for (int64_t node : path) blocks.push_back(nodes_[node].block);
  Status s = pool.adopt(seq, blocks.data(), static_cast<int32_t>(blocks.size()), h, msg);
  if (s == kOk) *hit = h;
  return s;
}

Status PrefixCache::add(BlockPool& pool, int64_t seq, const std::string& scope, const std::string& revision,
                        const int32_t* tokens, int64_t n, int64_t* added, std::string* msg) {
  const Sequence* s = pool.find(seq);
  if (!s) {
    *msg = "unknown sequence: " + std::to_string(seq);
    return kUnknownSeq;
  }
  if (n < 0 || n > s->length || (n > 0 && !tokens)) {
    *msg = "n_tokens must be in 0..length(seq) with non-NULL tokens";
    return kInvalidArg;
  }
  if (block_size_ != 0 && block_size_ != pool.block_size()) {
    *msg = "prefix cache bound to another block size";
    return kInvalidArg;
  }
  block_size_ = pool.block_size();
  // Keys stop at the first page a window released (its block is gone).
  for (int64_t j = 0; j < n / block_size_; ++j)
    if (s->table[j] == kHole) {
      n = j * block_size_;
      break;
    }
  const std::string rk = root_key(scope, revision);
  auto r = roots_.find(rk);
  if (r == roots_.end()) r = roots_.emplace(rk, static_cast<int64_t>(roots_.size())).first;
  int64_t parent = -(r->second + 1);
  int64_t count = 0;
  for (int64_t end = block_size_; end <= n; end += block_size_) {
    Edge e{parent, std::vector<int32_t>(tokens + end - block_size_, tokens + end)};
    auto it = edges_.find(e);
    if (it != edges_.end()) {
      parent = it->second;
      continue;
    }
    const int32_t block = s->table[end / block_size_ - 1];
    Status ps = pool.pin(block, msg);  // the block is in a live table: cannot fail
    if (ps != kOk) return ps;
    const int64_t id = static_cast<int64_t>(nodes_.size());
    nodes_.push_back({block});
    edges_.emplace(std::move(e), id);
    parent = id;
    ++count;
  }
  *added = count;
  return kOk;
}

int64_t PrefixCache::clear(BlockPool& pool) {
  const int64_t n = size();
  std::string msg;
  for (const Node& node : nodes_) (void)pool.unpin(node.block, &msg);
  nodes_.clear();
  edges_.clear();
  roots_.clear();
  return n;
}

}  // namespace pa
