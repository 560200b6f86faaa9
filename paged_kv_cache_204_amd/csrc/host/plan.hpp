// Host planners for the attention calls (no HIP in here).
//
// Decode: the batch's block tables are grouped into a trie keyed by physical
// block id, compressed into segments -- maximal runs of blocks that one set of
// queries shares.  This mirrors the radix-tree view of shared prefixes
// (SGLang RadixAttention page, "Mathematical and data-structure foundations"
// and the match / split operations), but keyed on blocks the pool already
// shares, so no token comparison is needed.  Each segment is read once per
// query group (all of the segment's queries x the GQA heads of one kv head)
// instead of once per query, split into key chunks for parallelism, and the
// partial softmax states are merged by log-sum-exp.
//
// Tree verify: one key range per sequence (context + draft-tree tail),
// split into chunks; the row groups are the tree nodes with their
// ancestor-or-self masks.
//
// Prefill: causal attention of a sequence's newest tokens, planned as
// windows of consecutive queries whose own tokens form a chain-shaped tail.
#pragma once

#include <string>
#include <vector>

#include "../plan_format.h"
#include "pool.hpp"

namespace pkv {

struct PlanConfig {
  int32_t valu_rows = 8;         // rows (groups x G) per VALU work item, <= 8
  int32_t valu_max_tokens = 512; // key tokens per VALU work item at most
  int32_t mfma_row_tiles = 0;    // 16-row tiles per wave of the MFMA path (1 or 2); 0 picks
                                 // 2 for calls with MFMA items only and 1 otherwise (the
                                 // two-tile kernel's registers lower the VALU items' occupancy)
  int32_t mfma_waves = 0;        // waves per MFMA workgroup (4 or 8); 0 picks 8 for calls
                                 // with MFMA items only whose query tiles fill 256 rows (one
                                 // K/V tile then feeds all of them), else 4
  int32_t mfma_min_rows = 32;    // segments with at least this many rows use MFMA; 0 = only
                                 // when a single query's GQA group exceeds valu_rows
  int32_t target_wgs = 256;      // VALU workgroups to aim for over all kv heads
  int32_t target_mfma_wgs = 512; // MFMA workgroups to aim for over all kv heads
  int32_t unshare_max_queries = 4;   // a shared run of at most this many queries ...
  int32_t unshare_max_tokens = 256;  // ... and tokens, too sparse for the MFMA path,
                                     // is read by each query's own item instead
  int32_t direct_max_tokens = 1024;  // decode calls whose queries all have at most this many
  int32_t direct_max_wgs = 768;      // keys, over at most this many (query, kv head) pairs,
                                     // run one workgroup per pair over all of its keys (no
                                     // partial states, no merge); 0 turns this off
  int32_t tile = 64;             // key tokens per kernel tile; chunks are multiples
  int32_t max_chunk = 4096;      // key tokens per work item at most
  int32_t max_parts = kMergeInline;  // partial states per query at most where the chunk
                                     // caps allow (beyond the merge row's inline list the
                                     // merge walks the parts serially); 0 = no limit
  int32_t wide_pairs = 1024;     // decode calls over at least this many (query, kv head)
  int32_t wide_max_parts = 6;    // pairs take at most this many partial states per query
                                 // (there is parallelism to spare: fewer, longer chunks
                                 // and a cheaper merge); 0 turns this off
  int32_t max_chunk_blocks = 512;// block ids per work item at most (LDS staging)
  int32_t mixed_kernel_only = 0; // 1: dense-tile-only plans at head_dim 128 run on the mixed
                                 // kernel too (at head_dim 64 they do anyway)
  // tree decode plans (block size >= 16): path items over the trie, very
  // long shared segments through MFMA items as partial states
  int32_t tree_decode = 1;       // 0 turns tree plans off
  int32_t tree_wide_rows = 1 << 20; // a segment read by at least this many rows ...
  int32_t tree_wide_tokens = 256;// ... and this many keys is shared through MFMA items
  int32_t tree_path_tokens = 4096; // longer segments always are
  int32_t tree_item_rows = 128;  // rows per MFMA item of a tree plan (16 .. 256)
  int32_t tree_target_wgs = 256; // MFMA workgroups to aim for over all kv heads
  int32_t tree_max_parts = 8;    // partial states per query at most (<= kPathMaxParts)
  int32_t tree_min_wgs = 128;    // path workgroups (items x kv heads) a tree plan needs
  int32_t private_segments = 0;  // 1: no trie, each decode query one segment over its table
                                 // (the smallest plan when a workspace is tight)
};

// Rows of one MFMA work item for a row-tile setting (4 waves x 16 x tiles).
inline int32_t mfma_item_rows(int32_t row_tiles, int32_t waves) { return waves * 16 * row_tiles; }

struct Plan {
  std::vector<WorkItem> valu;   // items for the VALU kernel
  std::vector<WorkItem> mfma;   // items for the MFMA kernel
  std::vector<WorkItem> direct; // one item per query for the direct kernel (then the only items)
  std::vector<RowGroup> groups;
  std::vector<int32_t> blocks;
  std::vector<MergeRow> merges;
  std::vector<int32_t> parts;
  std::vector<int32_t> item_blocks;   // per-item block lists, fixed strides
  // tree decode plans: path items and their steps (MFMA items above write
  // partial states in a launch before the path items', which merge them;
  // no merge launch)
  bool tree = false;
  std::vector<PathItem> paths;
  std::vector<PathStep> steps;
  int32_t stride_mfma = 0, stride_valu = 0, stride_direct = 0;
  int64_t partial_rows = 0;
  int32_t mfma_row_tiles = 1;   // row tiles per wave the MFMA items were cut for
  int32_t mfma_waves = 4;       // waves per MFMA workgroup (8 only without VALU items)
  int32_t valu_max_rows = 0;    // most rows in any VALU item
  // what the call reads
  int64_t unique_tokens = 0;
  int64_t logical_tokens = 0;
  int32_t unique_blocks = 0;
  int32_t segments = 0;
  // decode plans: each query's table epoch and length when planned, and the
  // items (launch order: MFMA, VALU, direct) that end at a query's last key
  std::vector<uint64_t> q_epoch;
  std::vector<int32_t> q_len;
  std::vector<int32_t> tail_items;

  // Empties the plan for reuse; the vectors keep their capacity, so
  // repeated planning of similar calls does not allocate.
  void reset() {
    valu.clear();
    mfma.clear();
    direct.clear();
    groups.clear();
    blocks.clear();
    merges.clear();
    parts.clear();
    item_blocks.clear();
    stride_mfma = stride_valu = stride_direct = 0;
    partial_rows = 0;
    mfma_row_tiles = 1;
    mfma_waves = 4;
    valu_max_rows = 0;
    unique_tokens = logical_tokens = 0;
    unique_blocks = segments = 0;
    q_epoch.clear();
    q_len.clear();
    tail_items.clear();
    tree = false;
    paths.clear();
    steps.clear();
  }
};

Err plan_decode(const BlockPool& pool, const int64_t* seqs, int32_t n_seqs,
                const PlanConfig& cfg, Plan* plan, std::string* why);

// The planners' last pass: each item's block list (plan.blocks from its
// blk_off) copied to a fixed stride per item kind in plan.item_blocks.
void pack_item_blocks(Plan* plan, int32_t block_size);

// Brings a decode plan for the same sequence list up to date without
// replanning when no table changed since it was made (same epochs) and the
// sequences only grew, i.e. appends filled their last blocks: the items that
// end at a query's last key take the new keys.  False (plan untouched) when
// that does not hold; the caller then plans afresh.
bool patch_decode(const BlockPool& pool, const int64_t* seqs, int32_t n_seqs, const PlanConfig& cfg,
                  Plan* plan);

// Tree decode plan of the call (its sequences already checked: known and
// non-empty).  False, with *plan untouched, when the call does not suit it
// (block size below 16, more than 16 query heads per kv head, a query that
// would need more partial states than tree_max_parts); the caller then
// plans segments and merges instead.
bool plan_tree(const BlockPool& pool, const int64_t* seqs, int32_t n_seqs, const PlanConfig& cfg,
               Plan* plan);

Err plan_verify(const BlockPool& pool, const int64_t* seqs, int32_t n_seqs,
                int32_t n_nodes, const int32_t* parent, const PlanConfig& cfg,
                Plan* plan, std::string* why);

// Most queries one prefill call takes (keeps query and partial-row indices
// in 32 bits).
constexpr int32_t kMaxPrefillQueries = 1 << 16;

// Causal attention of each sequence's newest tokens (a prompt's part that
// missed the prefix cache, appended already): the last n_new[i] tokens of
// sequence i are queries q_off[i] + j (q_off = running sum of n_new), and
// query j sees keys 0 .. len - n_new[i] + j.  n_new[i] may be 0.
Err plan_prefill(const BlockPool& pool, const int64_t* seqs, int32_t n_seqs, const int32_t* n_new,
                 const PlanConfig& cfg, Plan* plan, std::string* why);

// Ancestor-or-self masks of one draft tree: anc[0] = 1,
// anc[i] = anc[parent[i]] | 1 << i.  False if parent[] is not a tree in node
// order (parent[0] == -1, 0 <= parent[i] < i) or n_nodes is outside 1..64.
bool ancestor_masks(const int32_t* parent, int32_t n_nodes, uint64_t* anc);

}  // namespace pkv
