// Block-granular radix-tree prefix cache over the block pool (host only).
//
// The tree maps token-id sequences to the pool blocks that hold their K/V
// (SGLang RadixAttention page, "Node and edge structure": a node is a branch
// point with a dictionary of children and a reference counter of the active
// requests using it; an edge holds a run of token ids together with the
// physical pages of those tokens; the root is the empty sequence).  Sharing
// is block-paged as on the Trellis page ("RadixAttention in Trellis": a
// session that shares a prefix acquires the existing blocks, refcount + 1,
// instead of allocating and recomputing them), so an edge always holds a
// whole number of blocks, children are keyed by their first block's tokens,
// and a match counts whole blocks only: a probe that differs from a cached
// prompt inside its last block shares every block but that one (the page's
// hit-rate ceiling (L/32 - 1) / (L/32) at 32-token blocks).
//
// Operations (SGLang page, the radix tree's core operations and its
// eviction policy):
//   match   - longest whole-block prefix of a prompt found in the tree; a
//             new pool sequence acquires those blocks (the caller appends and
//             prefills only the rest) and every node on the path is locked
//             (lock + 1) and stamped with the access clock;
//   insert  - a sequence's whole blocks under its tokens; an edge that
//             diverges part-way is split at the block boundary into a parent
//             holding the common blocks and the old remainder as its child
//             (the blocks are re-sliced, never copied; the parent takes the
//             child's locks, and a live match that ended before the cut no
//             longer locks the remainder); new tokens become a leaf whose
//             blocks the cache references (refcount + 1);
//   release - the request that matched is done: lock - 1 along its path;
//             the blocks stay cached for later requests;
//   evict   - while the free list is short of a target: drop the unlocked
//             leaf with the oldest access stamp (the cache's references on
//             its blocks go, blocks reaching refcount 0 return to the free
//             list); a parent left without children becomes a candidate.
// Access stamps come from a counter bumped per touched node, so ties never
// occur and runs are deterministic.
#pragma once

#include <cstdint>
#include <map>
#include <memory>
#include <string>
#include <unordered_map>
#include <vector>

#include "pool.hpp"

namespace pkv {

struct RadixNode {
  std::vector<int32_t> tokens;   // the edge into this node: blocks.size() * B token ids
  std::vector<int32_t> blocks;   // pool block of each B tokens of the edge
  RadixNode* parent = nullptr;
  // children keyed by the tokens of their edge's first block
  std::map<std::vector<int32_t>, std::unique_ptr<RadixNode>> children;
  int32_t lock = 0;              // live matches whose path runs through this node
  uint64_t last_access = 0;
};

class RadixCache {
 public:
  explicit RadixCache(BlockPool* pool);
  ~RadixCache();   // drops the cache's block references (unless detached)
  // The pool goes away first: forget it; the destructor then drops nothing.
  void detach() { pool_ = nullptr; }
  bool attached() const { return pool_ != nullptr; }
  RadixCache(const RadixCache&) = delete;
  RadixCache& operator=(const RadixCache&) = delete;

  // New sequence holding the longest cached whole-block prefix of tokens[0..n).
  Err match(const int32_t* tokens, int32_t n, int64_t* seq, int32_t* matched, std::string* why);
  // Cache the whole blocks of `seq` under tokens[0..n) (n <= the sequence's length).
  Err insert(int64_t seq, const int32_t* tokens, int32_t n, std::string* why);
  // Unlock the path a match locked for `seq`.
  Err release(int64_t seq, std::string* why);
  // Evict until the free list holds want_free blocks; false if it cannot.
  bool evict(int32_t want_free);

  int32_t nodes() const { return n_nodes_; }
  int32_t cached_blocks() const { return n_blocks_; }
  int32_t locked_nodes() const;
  // Preorder over the tree (children in key order, root excluded):
  // depth, token count, lock, tokens..., blocks... per node.
  void dump(std::vector<int32_t>* out) const;

 private:
  void touch(RadixNode* n) { n->last_access = ++clock_; }
  RadixNode* split(RadixNode* child, int32_t keep_blocks);
  const BlockPool& cpool() const { return *pool_; }

  BlockPool* pool_;
  RadixNode root_;
  uint64_t clock_ = 0;
  int32_t n_nodes_ = 0;
  int32_t n_blocks_ = 0;
  // sequence -> the deepest node its match locked and how many of that
  // node's edge tokens it matched (a split moves the lock up when the match
  // ended before the cut)
  struct Held {
    RadixNode* node;
    int32_t reach;
  };
  std::unordered_map<int64_t, Held> matched_;
};

}  // namespace pkv
