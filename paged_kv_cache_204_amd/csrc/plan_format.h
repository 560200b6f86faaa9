// Work description that the host planner writes and the attention kernels
// read.  Plain structs, identical layout on host and device.
//
// A work item is an attention call's share for one workgroup per kv head
// (the launch runs every item once for each kv head):
//   - keys: n_tok tokens read through the item's block list (token t sits in
//     block list[t / B] at slot t % B).  The device copy of the lists has a
//     fixed stride per item kind (item_blocks below), so a workgroup finds
//     its list from its own index, without waiting for the item;
//   - queries: n_grp row groups from plan.groups[grp_off ...]; a row group is
//     one query vector (a decode query or a draft-tree node) and expands to
//     the G = Hq / Hkv query heads that read this kv head;
//   - tokens at relative index >= tail_start are draft-tree tokens: token
//     tail_start + k is tree node tail_node0 + k and a row sees it only if
//     that node is in the row's ancestor-or-self mask;
//   - output: part_base < 0 -> the item covers every key of its queries and
//     writes final out / lse; otherwise it writes normalised partial states
//     (o, lse) at partial rows part_base + u * Hq + hq (u = group index
//     within the item) for the merge launch.
#pragma once

#include <stdint.h>

namespace pkv {

struct WorkItem {
  int32_t blk_off;   // host side: the list at plan.blocks[blk_off ...]
  int32_t n_tok;
  int32_t tail_start;
  int32_t tail_node0;
  int32_t grp_off;
  int32_t n_grp;
  int32_t part_base;
  int32_t tail_q;    // host side: 1 + the query whose last key ends this item, else 0
  // query vectors of the first min(n_grp, 8) row groups, so the query loads
  // need only the item itself
  int32_t q_index[8];
};

struct RowGroup {
  int32_t q_index;   // query vector index: q + q_index * Hq * D, out likewise
  int32_t node;      // draft-tree node of this query, -1 for decode
  uint32_t anc_lo;   // ancestor-or-self mask of the node, bits 0..31
  uint32_t anc_hi;   // bits 32..63
  int32_t merge;     // MergeRow of this query, -1 when it has a single partial state
  int32_t pad[3];
};

// One query vector whose partial states are merged: partial rows
// part[p] + hq for p < n_parts, where part[] is inl[] when n_parts <=
// kMergeInline and parts[parts_off ...] otherwise.
constexpr int kMergeInline = 12;

struct MergeRow {
  int32_t q_index;
  int32_t n_parts;
  int32_t parts_off;
  int32_t pad;
  int32_t inl[kMergeInline];
};

// Narrow part of a tree decode plan: one path item per group of up to 32
// rows (queries x G, whole queries) that covers every key of its queries
// outside the shared segments given to MFMA items, step by step; each step
// is 32 consecutive tokens of one segment, seen by the item's queries in
// qmask.  The item merges its own softmax states with its queries' partial
// states from the MFMA items (a launch before it) and writes out / lse.
constexpr int kPathMaxQ = 32;
constexpr int kPathMaxRows = 32;   // two 16-row tiles
constexpr int kPathMaxParts = 8;   // partial states per query of a tree plan at most

struct PathItem {
  int32_t step_off;            // first step in the plan's step list
  int32_t n_steps;
  int32_t n_q;                 // queries of the item (q_index[0 .. n_q)), n_q * G <= kPathMaxRows
  int32_t pad;
  int32_t q_index[kPathMaxQ];
  int32_t merge[kPathMaxQ];    // MergeRow listing query j's partial states, -1 when none
};

struct PathStep {
  int32_t blk_a;               // block holding the step's tokens 0..15
  int32_t blk_b;               // block holding tokens 16..31 (blk_a when block_size >= 32)
  int32_t meta;                // bits 0..7: slot of token 0 in blk_a; bits 8..15: tokens (1..32)
  uint32_t qmask;              // bit j: query j of the item sees these tokens
};

// Device block lists: MFMA item i (kernel order) reads
// item_blocks[i * stride_mfma ...], VALU item j reads
// item_blocks[n_mfma * stride_mfma + j * stride_valu ...]; entries past an
// item's last block repeat that block.

static_assert(sizeof(WorkItem) == 64, "WorkItem layout");
static_assert(sizeof(RowGroup) == 32, "RowGroup layout");
static_assert(sizeof(MergeRow) == 64, "MergeRow layout");
static_assert(sizeof(PathItem) == 272, "PathItem layout");
static_assert(sizeof(PathStep) == 16, "PathStep layout");

}  // namespace pkv
