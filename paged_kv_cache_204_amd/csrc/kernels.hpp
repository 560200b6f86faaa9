// Launch parameters and launchers of the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan_format.h"

namespace pkv {

constexpr float kLog2eHost = 1.4426950408889634f;

// Copy-on-write copies plus the scatter of new K/V into their slots.
struct AppendParams {
  const uint16_t* k_new;  // [L][n_rows][Hkv][D], n_rows = n_seqs * n_tok
  const uint16_t* v_new;
  uint16_t* k_pool;       // [L][N][Hkv][B][D]
  uint16_t* v_pool;
  const int32_t* slots;   // [n_rows] block * B + offset
  const int32_t* cow;     // [n_cow][3] (src, dst, filled slots)
  int32_t n_rows;
  int32_t n_cow;
  int32_t L, N, Hkv, B, log2B, D;
};

// One attention launch over a list of work items, each run once per kv head:
// items [0, n_mfma) take the MFMA path, the rest the VALU path.
constexpr int kMaxItemBlocks = 512;   // block ids of one work item (LDS staging)
constexpr int kValuMaxRows = 8;       // query rows of one VALU work item
constexpr int kValuMaxTokens = 512;   // key tokens of one VALU work item (LDS scores)

struct AttnParams {
  const WorkItem* items;
  const RowGroup* groups;
  const int32_t* blocks;   // per-item block lists at fixed strides
  const uint16_t* q;       // [n_q][Hq][D]
  const uint16_t* k_pool;  // [L][N][Hkv][B][D]
  const uint16_t* v_pool;
  float* out;              // [n_q][Hq][D]
  float* lse;              // [n_q][Hq] natural log, or null
  float* part_o;           // [partial rows][D]
  float* part_lse;         // [partial rows], base-2 log
  int32_t n_mfma;
  int32_t stride_mfma, stride_valu;   // block-list stride of each item kind
  int32_t layer, N, Hq, Hkv, G, B, log2B;
  uint32_t g_magic;        // ceil(2^16 / G): r / G == (r * g_magic) >> 16 for r < 1024
  float scale_log2;        // sm_scale * log2(e)
  // tree decode plans: the path items' steps and the merge rows of their
  // queries' partial states
  const PathStep* steps;
  const MergeRow* merges;
  // direct launches over several layers: one layer of a pool in 16-byte
  // chunks, and the query (out) rows of one layer (queries x Hq)
  uint64_t layer_chunks;
  uint64_t layer_rows;
};

hipError_t launch_append(const AppendParams& p, hipStream_t s);

// 4-bit pools: codes u8 [L][N][Hkv][B][D/2] (two 4-bit codes per byte, the
// lower dim in the low nibble) and fp16 norms [L][N][Hkv][B], for K and V.

struct Q4AppendParams {
  const uint16_t* k_new;   // [L][n_rows][Hkv][D] bf16
  const uint16_t* v_new;
  uint8_t* k_codes;
  uint8_t* v_codes;
  uint16_t* k_norms;
  uint16_t* v_norms;
  const float* signs;      // [D] +-1
  const int32_t* slots;    // [n_rows] block * B + offset
  const int32_t* cow;      // [n_cow][3] (src, dst, filled slots)
  int32_t n_rows, n_cow;
  int32_t L, N, Hkv, B, log2B, D;
};

struct Q4Item {
  int32_t blk_off;   // the query's table at blocks[blk_off ...]
  int32_t n_tok;     // keys
  int32_t q_index;   // query vector (q, out, lse rows)
  int32_t pad;
};

struct Q4DecodeParams {
  const Q4Item* items;
  const int32_t* blocks;
  const uint16_t* q;       // [n][Hq][D] bf16
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const uint16_t* k_norms;
  const uint16_t* v_norms;
  const float* signs;
  float* out;              // [n][Hq][D]
  float* lse;              // [n][Hq] or null
  int32_t layer, N, Hq, Hkv, G, B, log2B;
  float scale_log2;
};

hipError_t launch_q4_append(const Q4AppendParams& p, hipStream_t s);

// Streaming read of `bytes` (16-byte aligned) by `blocks` workgroups of 256.
hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t blocks, hipStream_t s);
// One workgroup per (item, kv head); head_dim 64 or 128, G <= 16.
hipError_t launch_q4_decode(const Q4DecodeParams& p, int32_t n_items, int32_t head_dim, hipStream_t s,
                            hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

// Draft-tree commit: per sequence, copy-on-write copies then token moves
// (physical slots block * B + offset), one thread per pool column.
struct CommitParams {
  uint16_t* k_pool;          // [L][N][Hkv][B][D]
  uint16_t* v_pool;
  const int32_t* cow;        // [n_cow][3] (src, dst, slots copied)
  const int32_t* move_src;   // [n_move] old slot of the kept token
  const int32_t* move_dst;   // [n_move] its new slot
  const int32_t* seq_cow;    // [n_seqs + 1] copies of sequence i: [seq_cow[i], seq_cow[i + 1])
  const int32_t* seq_move;   // [n_seqs + 1] likewise for moves
  int32_t seq0;              // first sequence of this launch
  int32_t L, N, Hkv, B, log2B, D;
};

// Sequences seq0 .. seq0 + n_seqs - 1 of the plan, side by side.
hipError_t launch_commit(const CommitParams& p, int32_t n_seqs, hipStream_t s);
// valu_rows: the most rows any VALU item of the launch holds (<= 8);
// waves: 4, or 8 for launches of MFMA items only (row_tiles 2).  Non-null
// events take the start and end times of the kernel's own dispatch.
hipError_t launch_attn(const AttnParams& p, int32_t n_items, int32_t head_dim, int32_t row_tiles,
                       int32_t valu_rows, int32_t waves, hipStream_t s, hipEvent_t ev_start = nullptr,
                       hipEvent_t ev_stop = nullptr);

// Dense tiles only (every item an MFMA item, up to 256 rows): one workgroup
// of 4, 8 or 16 waves per (item, kv head), software-pipelined steps;
// items[i]'s block list at blocks + i * stride (<= kMaxItemBlocks);
// max_rows: the most rows (row groups x G) of any item, 1..256.
// no_scratch: only kernels that use no private (scratch) memory -- the
// sixteen-wave variant spills a few registers, and the runtime sizes a
// queue's scratch area at the first launch that needs it.
hipError_t launch_wide(const AttnParams& p, int32_t n_items, int32_t head_dim, int32_t stride,
                       int32_t max_rows, hipStream_t s, hipEvent_t ev_start = nullptr,
                       hipEvent_t ev_stop = nullptr, bool no_scratch = false);

// Path items of a tree decode plan: one workgroup of eight waves per (path
// item, kv head); the waves take the item's steps (p.steps) in turn, then
// combine their states with the queries' partial states from the MFMA items
// (p.merges, p.part_o / part_lse, written by an earlier launch) and write
// out / lse.
hipError_t launch_path(const AttnParams& p, const PathItem* items, int32_t n_items, int32_t head_dim,
                       hipStream_t s, hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

// Direct decode: one workgroup per (item, kv head), each item one query
// over all of its keys (n_grp 1, tail_start INT_MAX), written straight to
// out / lse; items[i]'s block list at blocks + i * stride (<= kMaxItemBlocks).
// max_tok: the largest n_tok of the items (it picks the kernel's form).
// n_layers > 1: the same items over layers p.layer .. p.layer + n_layers - 1
// in one launch (grid z), layer z's q / out / lse rows at z * p.layer_rows
// and its pool data at z * p.layer_chunks past layer p.layer's.
hipError_t launch_direct(const AttnParams& p, int32_t n_items, int32_t head_dim, int32_t stride,
                         int32_t max_tok, hipStream_t s, hipEvent_t ev_start = nullptr,
                         hipEvent_t ev_stop = nullptr, int32_t n_layers = 1);

// Log-sum-exp merge of the partial states of several work items.
struct MergeParams {
  const MergeRow* merges;
  const int32_t* parts;
  const float* part_o;
  const float* part_lse;   // base-2
  float* out;
  float* lse;              // natural log, or null
  int32_t Hq, D;
};
hipError_t launch_merge(const MergeParams& p, int32_t n_rows, hipStream_t s);

}  // namespace pkv
