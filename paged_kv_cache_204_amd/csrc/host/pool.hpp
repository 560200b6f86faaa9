// Host side of the refcounted, copy-on-write block pool.  No HIP in here:
// this builds and runs on a CPU-only machine.
//
// Rules (Dendrite page, section details and glossary "Copy-on-Write";
// "Introducing RadixAttention into Trellis", section "RadixAttention in
// Trellis"; SGLang RadixAttention page, source-level sketch of the free page
// pool):
//   fork   - child table = parent table, refcount + 1 per block;
//   free   - refcount - 1 per block in table order, zero -> tail of free list;
//   append - per sequence in call order, per token: len % B == 0 -> fresh
//            block from the free-list head; else if the last block is shared
//            (refcount > 1) -> copy its filled slots into a fresh block and
//            drop one reference from the original; write the token at
//            (table[len / B], len % B).  All-or-nothing.
#pragma once

#include <cstdint>
#include <deque>
#include <string>
#include <unordered_map>
#include <vector>

namespace pkv {

enum class Err : int {
  ok = 0,
  arg = -1,
  oom = -2,
  seq = -3,
  hip = -4,
  empty = -5,
  unsupported = -6,
};

struct Shape {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  int32_t num_layers = 0;
  int32_t num_q_heads = 0;
  int32_t num_kv_heads = 0;
  int32_t head_dim = 0;
};

// Check a shape for a pool; fills `why` on failure.
bool valid_shape(const Shape& s, std::string* why);

struct SeqState {
  std::vector<int32_t> table;
  int32_t len = 0;
  // Changes whenever the table does (allocate, fork, an append that adds or
  // replaces a block), never when an append only fills the last block;
  // unique over the pool's life, so a reused id never repeats one.
  uint64_t epoch = 0;
};

struct CowCopy {
  int32_t src;
  int32_t dst;
  int32_t n_slots;  // filled slots copied: [0, n_slots)
};

struct AppendResult {
  std::vector<int32_t> slots;  // [n_seqs * n_tok] physical slot = block * B + off
  std::vector<CowCopy> cow;    // in the order taken
};

// An append worked out against the current state but not applied yet.
struct PendingAppend {
  AppendResult result;
  std::vector<std::pair<int64_t, SeqState>> states;     // new state of each sequence
  std::vector<std::pair<int32_t, int32_t>> refcounts;   // final refcount of each touched block
  size_t taken = 0;                                     // blocks taken from the free-list head
  uint64_t version = 0;                                 // pool version it was computed on
};

// A draft-tree commit worked out against the current state (see
// BlockPool::prepare_commit).  Token moves are physical slots
// (block * B + offset): the source in the sequence's old table, the
// destination in its new one.
struct PendingCommit {
  std::vector<std::pair<int64_t, SeqState>> states;
  std::vector<std::pair<int32_t, int32_t>> refcounts;  // final refcount of each touched block
  std::vector<int32_t> pushed;   // blocks released to the free-list tail, in order
  size_t taken = 0;              // taken from the head (blocks free before the call)
  std::vector<CowCopy> cow;      // all sequences' copies, in order
  std::vector<int32_t> move_src, move_dst;
  std::vector<int32_t> seq_cow;  // per sequence: first copy, one past the last at [i + 1]
  std::vector<int32_t> seq_move; // per sequence: first move, likewise
  bool conflict = false;         // a sequence writes in place a block another one reads
  uint64_t version = 0;
};

class BlockPool {
 public:
  BlockPool(const Shape& s, const int32_t* free_order);

  const Shape& shape() const { return shape_; }
  int32_t log2_block() const { return log2b_; }

  int64_t allocate();
  Err fork(int64_t parent, int64_t* child, std::string* why);
  Err release(int64_t seq, std::string* why);

  // Work out an append without changing anything; commit_append applies it.
  // Errors (unknown or repeated sequence, exhausted pool) leave no trace.
  Err prepare_append(const int64_t* seqs, int32_t n_seqs, int32_t n_tok,
                     PendingAppend* out, std::string* why) const;
  // Apply a prepared append (must be the next change to the pool).
  void commit_append(PendingAppend&& pa);

  // Keep the accepted path of each sequence's draft tree (its last n_nodes
  // tokens, node order; parent [n_seqs][n_nodes]; path i = paths[i *
  // n_nodes ...], path_len[i] nodes, root first along parent links) and drop
  // the rest.  Per sequence in call order: blocks past the new length go
  // back (table order), then every shared block that receives a moved
  // token is copied first (copy-on-write, table order).  Nothing changes
  // until commit_commit; errors leave no trace.
  Err prepare_commit(const int64_t* seqs, int32_t n_seqs, int32_t n_nodes, const int32_t* parent,
                     const int32_t* path_len, const int32_t* paths, PendingCommit* out,
                     std::string* why) const;
  void commit_commit(PendingCommit&& pc);

  // A new sequence over existing blocks (a prefix-cache hit): its table is
  // `blocks`, its length `len`, and every block gains a reference.  `len`
  // must lie in ((n_blocks - 1) * B, n_blocks * B] (0 with no blocks) and
  // every block must be held already.
  Err adopt(const int32_t* blocks, int32_t n_blocks, int32_t len, int64_t* seq, std::string* why);
  // A reference held outside any sequence (the prefix cache's own), taken
  // on a held block / dropped (zero -> tail of the free list).
  void retain(int32_t block);
  void drop(int32_t block);

  const SeqState* find(int64_t seq) const;
  int32_t refcount(int32_t block) const { return rc_[block]; }
  const std::deque<int32_t>& free_list() const { return fifo_; }

  // Bumped by every change to tables or refcounts (plans keyed on it).
  uint64_t version() const { return version_; }

  const AppendResult& last_append() const { return last_append_; }

 private:
  Shape shape_;
  int32_t log2b_ = 0;
  std::vector<int32_t> rc_;
  std::deque<int32_t> fifo_;
  std::unordered_map<int64_t, SeqState> seqs_;
  int64_t next_id_ = 0;
  uint64_t version_ = 0;
  uint64_t epochs_ = 0;
  AppendResult last_append_;
};

}  // namespace pkv
