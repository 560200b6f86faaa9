// Work description that the host planner writes and the attention kernels
// read.  Plain structs, identical layout on host and device.
//
// A work item is one workgroup's share of an attention call for one kv head
// (the kv head is blockIdx.y):
//   - keys: n_tok tokens read through plan.blocks[blk_off ...] (token t sits
//     in block blocks[blk_off + t / B] at slot t % B);
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
  int32_t blk_off;
  int32_t n_tok;
  int32_t tail_start;
  int32_t tail_node0;
  int32_t grp_off;
  int32_t n_grp;
  int32_t part_base;
  int32_t xcd_slot;  // informational: the XCD the planner aimed this item at
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
// parts[parts_off + p] + hq for p < n_parts.
struct MergeRow {
  int32_t q_index;
  int32_t parts_off;
  int32_t n_parts;
  int32_t pad;
};

static_assert(sizeof(WorkItem) == 32, "WorkItem layout");
static_assert(sizeof(RowGroup) == 32, "RowGroup layout");
static_assert(sizeof(MergeRow) == 16, "MergeRow layout");

}  // namespace pkv
