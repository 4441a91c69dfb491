// Prefix-hash block reuse over a BlockPool.
//
// Keys follow the vladkulikov.com notebook "Модуль 10" (prefix-caching
// cell): a key exists only at a complete block boundary and is (scope,
// revision, every token id before the boundary); a request's hit is the
// longest run of consecutive cached complete blocks from the first block.
//
// Representation: a key for boundary `end` is identified exactly by the key
// for `end - block_size` plus the block's own token ids, so the cache is a
// trie with one root per (scope, revision) and one node per cached complete
// block; each node holds one pin on the physical block that stores it.
// Equal keys are equal paths, compared token by token (no hash collisions).
#pragma once

#include <cstdint>
#include <string>
#include <unordered_map>
#include <vector>

#include "pool.hpp"

namespace pa {

class PrefixCache {
 public:
  // Tokens covered by the longest run of cached complete blocks of tokens[0..n).
  int64_t lookup(const std::string& scope, const std::string& revision, const int32_t* tokens,
                 int64_t n) const;
  // New sequence `seq` holding the cached blocks of its hit (pool.adopt);
  // *hit receives the hit in tokens.  Errors: kSeqExists, kInvalidArg.
  Status attach(BlockPool& pool, int64_t seq, const std::string& scope, const std::string& revision,
                const int32_t* tokens, int64_t n, int64_t* hit, std::string* msg);
  // Add the keys of the complete blocks of `seq`'s first n tokens (token ids
  // tokens[0..n), n <= length), up to the first page a window released; a
  // key already cached keeps its block.
  // *added receives the number of new keys (each pins its block).
  Status add(BlockPool& pool, int64_t seq, const std::string& scope, const std::string& revision,
             const int32_t* tokens, int64_t n, int64_t* added, std::string* msg);
  // Drop every key and its pin; returns how many keys there were.
  int64_t clear(BlockPool& pool);
  int64_t size() const { return static_cast<int64_t>(nodes_.size()); }

 private:
  struct Edge {
    int64_t parent;               // node id, or -(root index + 1) for a root
    std::vector<int32_t> tokens;  // the block's token ids
    bool operator==(const Edge& o) const { return parent == o.parent && tokens == o.tokens; }
  };
  struct EdgeHash {
    size_t operator()(const Edge& e) const;
  };
  struct Node {
    int32_t block;
  };
  static std::string root_key(const std::string& scope, const std::string& revision);
  // Walk from the root of (scope, revision); returns the hit and fills the
  // node ids passed (one per cached block).
  int64_t walk(const std::string& scope, const std::string& revision, const int32_t* tokens, int64_t n,
               int32_t block_size, std::vector<int64_t>* path) const;

  int32_t block_size_ = 0;  // fixed by the first add
  std::unordered_map<std::string, int64_t> roots_;
  std::unordered_map<Edge, int64_t, EdgeHash> edges_;
  std::vector<Node> nodes_;
};

}  // namespace pa
