// C ABI: the calls declared in include/pkv.h.
//
// Host metadata lives in pkv::BlockPool (tables, refcounts, free list) and
// the planners; this file adds the device side: the pool's own scratch
// (plan buffers, partial softmax states), a small ring of pinned staging
// buffers for plan uploads, and the kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "pkv.h"
#include "host/plan.hpp"
#include "host/radix.hpp"
#include "host/pool.hpp"
#include "kernels.hpp"

namespace {

thread_local std::string g_err;

pkv_status fail(pkv_status s, std::string msg) {
  g_err = std::move(msg);
  return s;
}

pkv_status to_status(pkv::Err e) { return static_cast<pkv_status>(static_cast<int>(e)); }

#define PKV_HIP(call)                                                                 \
  do {                                                                                \
    hipError_t e_ = (call);                                                           \
    if (e_ != hipSuccess)                                                             \
      return fail(PKV_ERR_HIP, std::string(#call) + ": " + hipGetErrorString(e_));    \
  } while (0)

struct DevBuf {
  void* ptr = nullptr;
  size_t cap = 0;
  bool owned = true;   // false: a region of the caller's workspace (never grown or freed)
};

constexpr int kStageSlots = 4;

size_t align16(size_t x) { return (x + 15) & ~size_t{15}; }

// Offsets of the plan arrays inside one contiguous upload.
struct PlanLayout {
  size_t items = 0, groups = 0, blocks = 0, merges = 0, parts = 0, paths = 0, steps = 0, total = 0;
};

PlanLayout layout_of(const pkv::Plan& p) {
  PlanLayout o;
  size_t at = 0;
  auto put = [&](size_t& field, size_t bytes) {
    field = at;
    at += align16(bytes);
  };
  put(o.items, (p.mfma.size() + p.valu.size() + p.direct.size()) * sizeof(pkv::WorkItem));
  put(o.groups, p.groups.size() * sizeof(pkv::RowGroup));
  put(o.blocks, p.item_blocks.size() * sizeof(int32_t));
  put(o.merges, p.merges.size() * sizeof(pkv::MergeRow));
  put(o.parts, p.parts.size() * sizeof(int32_t));
  put(o.paths, p.paths.size() * sizeof(pkv::PathItem));
  put(o.steps, p.steps.size() * sizeof(pkv::PathStep));
  o.total = at;
  return o;
}

void serialize(const pkv::Plan& p, const PlanLayout& o, char* dst) {
  auto cp = [&](size_t off, const void* src, size_t bytes) {
    if (bytes) std::memcpy(dst + off, src, bytes);
  };
  // MFMA items first: the kernel picks its path by block index
  cp(o.items, p.mfma.data(), p.mfma.size() * sizeof(pkv::WorkItem));
  cp(o.items + p.mfma.size() * sizeof(pkv::WorkItem), p.valu.data(), p.valu.size() * sizeof(pkv::WorkItem));
  cp(o.items + (p.mfma.size() + p.valu.size()) * sizeof(pkv::WorkItem), p.direct.data(),
     p.direct.size() * sizeof(pkv::WorkItem));
  cp(o.groups, p.groups.data(), p.groups.size() * sizeof(pkv::RowGroup));
  cp(o.blocks, p.item_blocks.data(), p.item_blocks.size() * sizeof(int32_t));
  cp(o.merges, p.merges.data(), p.merges.size() * sizeof(pkv::MergeRow));
  cp(o.parts, p.parts.data(), p.parts.size() * sizeof(int32_t));
  cp(o.paths, p.paths.data(), p.paths.size() * sizeof(pkv::PathItem));
  cp(o.steps, p.steps.data(), p.steps.size() * sizeof(pkv::PathStep));
}

// Makes the pool's device current for the duration of a call.
struct DeviceGuard {
  int prev = -1;
  bool changed = false;
  hipError_t err = hipSuccess;
  explicit DeviceGuard(int dev) {
    err = hipGetDevice(&prev);
    if (err == hipSuccess && prev != dev) {
      err = hipSetDevice(dev);
      changed = err == hipSuccess;
    }
  }
  ~DeviceGuard() {
    if (changed) (void)hipSetDevice(prev);
  }
};

}  // namespace

struct pkv_radix;

struct pkv_pool {
  explicit pkv_pool(const pkv::Shape& s, const int32_t* order) : core(s, order) {}
  std::vector<pkv_radix*> radixes;   // live prefix caches over this pool
  pkv::BlockPool core;
  pkv::PlanConfig cfg;
  bool device = false;
  int dev = -1;
  uint16_t* k_pool = nullptr;
  uint16_t* v_pool = nullptr;
  DevBuf append_plan, commit_plan, decode_plan, verify_plan, prefill_plan, partials;
  // a caller workspace: the four buffers above from decode_plan on are its
  // fixed regions, and calls stay within these limits
  bool ws_fixed = false;
  int32_t ws_max_seqs = 0, ws_max_nodes = 0;
  // outgrown buffers of the pool's own, freed once their event has completed
  std::vector<std::pair<void*, hipEvent_t>> retired;
  // 4-bit pools: codes and norms instead of bf16 K/V (k_pool / v_pool unused)
  bool q4 = false;
  uint8_t* k_codes = nullptr;
  uint8_t* v_codes = nullptr;
  uint16_t* k_norms = nullptr;
  uint16_t* v_norms = nullptr;
  DevBuf signs;   // float [head_dim], +-1
  std::vector<pkv::Q4Item> q4_items;
  std::vector<int32_t> q4_blocks;
  void* stage[kStageSlots] = {};
  size_t stage_cap[kStageSlots] = {};
  hipEvent_t stage_ev[kStageSlots] = {};
  bool stage_used[kStageSlots] = {};
  int stage_next = 0;
  // decode plan cache: same sequence list on an unchanged pool -> reuse;
  // after appends that only filled the last blocks -> patch (patch_decode)
  bool dcache_valid = false;
  uint64_t dcache_version = 0;
  std::vector<int64_t> dcache_seqs;
  pkv::Plan dplan;
  PlanLayout dlayout;
  pkv::Plan vplan;
  PlanLayout vlayout;
  // verify plan cache: the same tree over the same sequences on an
  // unchanged pool (every layer of one verify step) reuses the uploaded plan
  bool vcache_valid = false;
  uint64_t vcache_version = 0;
  int32_t vcache_nodes = 0;
  std::vector<int64_t> vcache_seqs;
  std::vector<int32_t> vcache_parent;
  // paged_attn_decode_scratch: its plan and the host copy it uploads from
  pkv::Plan splan;
  PlanLayout slayout;
  std::vector<char> sstage;
  // prefill plan cache: the same call repeated at every layer of a step
  // (same sequences and counts, pool unchanged) reuses the uploaded plan
  bool pcache_valid = false;
  uint64_t pcache_version = 0;
  std::vector<int64_t> pcache_seqs;
  std::vector<int32_t> pcache_new;
  pkv::Plan pplan;
  PlanLayout playout;
  // kernel timing: event pairs recorded around every timing_every-th
  // attention kernel
  bool timing = false;
  int32_t timing_every = 1;
  int64_t timing_tick = 0;
  std::vector<hipEvent_t> ev_free;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev_pending;
  double timed_ms = 0.0;
  int64_t timed_calls = 0;
};

struct pkv_radix {
  explicit pkv_radix(pkv_pool* p) : pool(p), cache(&p->core) {}
  pkv_pool* pool;          // null once the pool was destroyed first
  pkv::RadixCache cache;
};

namespace {
// A pool destroyed before its caches: they forget it (their later calls
// fail, radix_destroy frees only the cache itself).
void detach_radixes(pkv_pool* p) {
  for (pkv_radix* r : p->radixes) {
    r->cache.detach();
    r->pool = nullptr;
  }
  p->radixes.clear();
}
}  // namespace


namespace {

// Frees the outgrown buffers whose last readers have finished.
void reap(pkv_pool* p) {
  for (size_t i = 0; i < p->retired.size();) {
    if (hipEventQuery(p->retired[i].second) == hipSuccess) {
      (void)hipFree(p->retired[i].first);
      (void)hipEventDestroy(p->retired[i].second);
      p->retired[i] = p->retired.back();
      p->retired.pop_back();
    } else {
      ++i;
    }
  }
}

// Room for `bytes` in b.  A region of the caller's workspace never grows
// (PKV_ERR_OOM); a buffer of the pool's own is replaced by a larger one and
// the old one kept until the work enqueued on `stream` so far has finished
// with it (an event; no device-wide synchronisation).
pkv_status ensure(pkv_pool* p, DevBuf& b, size_t bytes, hipStream_t stream) {
  if (bytes <= b.cap) return PKV_OK;
  if (!b.owned)
    return fail(PKV_ERR_OOM, "a workspace region of " + std::to_string(b.cap) + " bytes cannot hold " +
                                 std::to_string(bytes));
  reap(p);
  const size_t want = bytes + bytes / 2 + 4096;
  void* np = nullptr;
  PKV_HIP(hipMalloc(&np, want));
  if (b.ptr) {
    hipEvent_t ev = nullptr;
    hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventRecord(ev, stream);
    if (e != hipSuccess) {
      if (ev) (void)hipEventDestroy(ev);
      (void)hipFree(np);
      return fail(PKV_ERR_HIP, std::string("ensure: ") + hipGetErrorString(e));
    }
    p->retired.emplace_back(b.ptr, ev);
  }
  b.ptr = np;
  b.cap = want;
  return PKV_OK;
}

// Copy `bytes` produced by `fill` into device buffer `dst` via a pinned
// staging slot, ordered on `stream`.  A slot is reused only after the copy
// that last read it has completed.
template <class Fill>
pkv_status upload(pkv_pool* p, DevBuf& dst, size_t bytes, hipStream_t stream, Fill fill) {
  pkv_status s = ensure(p, dst, bytes, stream);
  if (s != PKV_OK) return s;
  if (bytes == 0) return PKV_OK;
  const int i = p->stage_next;
  p->stage_next = (i + 1) % kStageSlots;
  if (p->stage_used[i]) PKV_HIP(hipEventSynchronize(p->stage_ev[i]));
  if (p->stage_cap[i] < bytes) {
    if (p->stage[i]) PKV_HIP(hipHostFree(p->stage[i]));
    p->stage[i] = nullptr;
    p->stage_cap[i] = 0;
    size_t want = bytes + bytes / 2 + 4096;
    PKV_HIP(hipHostMalloc(&p->stage[i], want, hipHostMallocDefault));
    p->stage_cap[i] = want;
  }
  if (!p->stage_ev[i]) PKV_HIP(hipEventCreateWithFlags(&p->stage_ev[i], hipEventDisableTiming));
  fill(static_cast<char*>(p->stage[i]));
  PKV_HIP(hipMemcpyAsync(dst.ptr, p->stage[i], bytes, hipMemcpyHostToDevice, stream));
  PKV_HIP(hipEventRecord(p->stage_ev[i], stream));
  p->stage_used[i] = true;
  return PKV_OK;
}

pkv_status take_event(pkv_pool* p, hipEvent_t* ev) {
  if (!p->ev_free.empty()) {
    *ev = p->ev_free.back();
    p->ev_free.pop_back();
    return PKV_OK;
  }
  PKV_HIP(hipEventCreate(ev));
  return PKV_OK;
}

size_t partial_bytes(const pkv::Plan& plan, const pkv::Shape& sh) {
  return static_cast<size_t>(plan.partial_rows) * (sh.head_dim + 1) * sizeof(float);
}

// ---- workspace ----------------------------------------------------------
//
// Regions for calls of at most S sequences and T query tokens per sequence,
// from what the planners can produce (N blocks of B tokens, Hq query heads):
//  - a work item's device entry is a WorkItem and a block list padded to
//    the plan's longest, at most min(512, N) blocks;
//  - the coarsest plan of a call (fit_plan: no shared runs, longest chunks)
//    cuts a sequence into at most c = ceil(N B / min(4096, 512 B)) items;
//  - a decode plan: up to 16 + c items and row groups per query, one merge
//    row, 64 overflow part ids, one path item and 64 steps per query (plus
//    65536 steps); up to max(12, c) partial states per query and head;
//  - verify / prefill: S T query rows in windows of at least one row, each
//    window up to max(4, c) items and partial states;
//  - 4-bit decode: an item and a whole block table per query.
constexpr size_t kWsAlign = 256;
constexpr int32_t kDefaultMaxSeqs = 256;
constexpr int32_t kDefaultMaxNodes = 64;

size_t ws_align(size_t x) { return (x + kWsAlign - 1) & ~(kWsAlign - 1); }

struct WsLayout {
  size_t decode = 0, verify = 0, prefill = 0, partials = 0, total = 0;
};

WsLayout ws_layout(const pkv::Shape& sh, int64_t S, int64_t T) {
  const int64_t N = sh.num_blocks, B = sh.block_size, Hq = sh.num_q_heads, D = sh.head_dim;
  const int64_t mb = std::min<int64_t>(512, N);
  const int64_t cap_tok = std::min<int64_t>(4096, 512 * B);
  const int64_t c = (N * B + cap_tok - 1) / cap_tok;
  const int64_t item = static_cast<int64_t>(sizeof(pkv::WorkItem)) + 4 * mb;
  const int64_t grp = sizeof(pkv::RowGroup), mrg = sizeof(pkv::MergeRow);
  const int64_t pad = 8 * 16;   // the plan arrays' 16-byte alignment
  WsLayout w;
  int64_t dec = S * (16 + c) * (item + grp) + S * mrg + S * 64 * 4 + S * static_cast<int64_t>(sizeof(pkv::PathItem)) +
                (64 * S + 65536) * static_cast<int64_t>(sizeof(pkv::PathStep)) + pad;
  dec = std::max<int64_t>(dec, S * static_cast<int64_t>(sizeof(pkv::Q4Item)) + S * N * 4 + pad);
  const int64_t Q = S * T;
  const int64_t pv = std::max<int64_t>(4, c);
  const int64_t ver = Q * pv * item + Q * grp + Q * mrg + Q * pv * 4 + pad;
  const int64_t rows = std::max(S * Hq * std::max<int64_t>(12, c), Q * Hq * pv);
  w.decode = ws_align(static_cast<size_t>(dec));
  w.verify = ws_align(static_cast<size_t>(ver));
  w.prefill = w.verify;
  w.partials = ws_align(static_cast<size_t>(rows * (D + 1) * 4));
  w.total = w.decode + w.verify + w.prefill + w.partials;
  return w;
}

// Planner settings for the smallest plan of a call: no tree or shared runs
// (a decode query is one segment, or one direct item), every item a dense
// tile, the longest chunks and so the fewest items and partial states.
pkv::PlanConfig coarse_config(const pkv::PlanConfig& cfg) {
  pkv::PlanConfig c = cfg;
  c.tree_decode = 0;
  c.private_segments = 1;
  c.direct_max_tokens = 1 << 30;
  c.direct_max_wgs = 1 << 30;
  c.mfma_min_rows = 1;
  c.max_parts = 1;
  c.target_wgs = 1;
  c.target_mfma_wgs = 1;
  c.max_chunk = 4096;
  c.max_chunk_blocks = 512;
  return c;
}

// Whether a plan's work lists fit `region` and its partial states the
// partial-state region; always true for a pool that grows its own buffers.
bool fits_workspace(const pkv_pool* p, const pkv::Plan& plan, const PlanLayout& lay, const DevBuf& region,
                    const DevBuf& parts) {
  if (region.owned && parts.owned) return true;
  return lay.total <= region.cap && partial_bytes(plan, p->core.shape()) <= parts.cap;
}

// Plans a call with the pool's settings and, when that plan does not fit a
// caller workspace, once more with coarse_config; PKV_ERR_OOM if neither fits.
template <class PlanWith>
pkv_status plan_to_fit(pkv_pool* p, const DevBuf& region, const DevBuf& parts, const char* what, pkv::Plan* plan,
                       PlanLayout* lay, PlanWith plan_with) {
  std::string why;
  pkv::Err e = plan_with(p->cfg, plan, &why);
  if (e != pkv::Err::ok) return fail(to_status(e), why);
  *lay = layout_of(*plan);
  if (fits_workspace(p, *plan, *lay, region, parts)) return PKV_OK;
  e = plan_with(coarse_config(p->cfg), plan, &why);
  if (e != pkv::Err::ok) return fail(to_status(e), why);
  *lay = layout_of(*plan);
  if (fits_workspace(p, *plan, *lay, region, parts)) return PKV_OK;
  return fail(PKV_ERR_OOM, std::string(what) + ": the call's work lists (" + std::to_string(lay->total) +
                               " bytes) or partial states (" +
                               std::to_string(partial_bytes(*plan, p->core.shape())) +
                               " bytes) do not fit the workspace regions (" + std::to_string(region.cap) +
                               " and " + std::to_string(parts.cap) + " bytes)");
}

// Every item must fit the tiles its kernel path assumes (LDS arrays, rows
// per workgroup); the planner guarantees it, this re-checks before launch.
bool plan_fits_kernels(const pkv::Plan& plan, const pkv::Shape& sh) {
  const int32_t G = sh.num_q_heads / sh.num_kv_heads;
  if (plan.tree) {
    // MFMA items of up to 256 rows writing partial states, path items of at
    // most 32 rows whose steps name pool blocks, merge rows of inline parts
    if (!plan.valu.empty() || !plan.direct.empty() || G > 16 || sh.block_size < 16) return false;
    for (const pkv::WorkItem& it : plan.mfma)
      if (it.n_tok < 1 || it.n_grp < 1 || it.n_grp * G > 256 || it.part_base < 0 ||
          it.tail_start != INT_MAX)
        return false;
    for (const pkv::MergeRow& m : plan.merges)
      if (m.n_parts < 1 || m.n_parts > pkv::kPathMaxParts) return false;
    const int64_t n_steps = static_cast<int64_t>(plan.steps.size());
    for (const pkv::PathItem& pi : plan.paths) {
      if (pi.n_q < 1 || pi.n_q > pkv::kPathMaxQ || pi.n_q * G > pkv::kPathMaxRows || pi.n_steps < 0 || pi.step_off < 0 ||
          pi.step_off + static_cast<int64_t>(pi.n_steps) > n_steps)
        return false;
      for (int32_t j = 0; j < pi.n_q; ++j)
        if (pi.merge[j] >= static_cast<int32_t>(plan.merges.size())) return false;
    }
    for (const pkv::PathStep& ps : plan.steps) {
      const int32_t n = (ps.meta >> 8) & 0xFF, off = ps.meta & 0xFF;
      // 16-token blocks: tokens 0..15 in blk_a, 16..31 in blk_b; larger
      // blocks: the step's tokens are slots off .. off + n - 1 of one block
      const bool in_block = sh.block_size == 16 ? off == 0 : (ps.blk_a == ps.blk_b && off + n <= sh.block_size);
      if (ps.blk_a < 0 || ps.blk_a >= sh.num_blocks || ps.blk_b < 0 || ps.blk_b >= sh.num_blocks ||
          n < 1 || n > 32 || !in_block)
        return false;
    }
    return true;
  }
  const int32_t mrows = pkv::mfma_item_rows(plan.mfma_row_tiles, plan.mfma_waves);
  if (plan.mfma_waves == 8 && !plan.valu.empty()) return false;
  for (const pkv::WorkItem& it : plan.valu)
    if (it.n_tok < 1 || it.n_tok > pkv::kValuMaxTokens || it.n_grp < 1 || it.n_grp * G > pkv::kValuMaxRows)
      return false;
  for (const pkv::WorkItem& it : plan.mfma)
    if (it.n_tok < 1 || it.n_grp < 1 || it.n_grp * G > mrows) return false;
  if (!plan.direct.empty()) {
    // a direct plan holds nothing else: the direct kernel numbers its items from 0
    if (!plan.mfma.empty() || !plan.valu.empty() || !plan.merges.empty() || G > 16) return false;
    for (const pkv::WorkItem& it : plan.direct)
      if (it.n_tok < 1 || it.n_grp != 1 || it.tail_start != INT_MAX) return false;
  }
  return true;
}

// The attention kernel of one call (the direct kernel for direct plans)
// and, when some queries have several partial states, the merge kernel.
// With timing enabled, a pair of events takes the attention kernel's own
// start and end.  no_scratch: only kernels without private (scratch)
// memory, whose first launch could make the runtime allocate.
pkv_status launch_plan(pkv_pool* p, const pkv::Plan& plan, const PlanLayout& lay,
                          const DevBuf& buf, DevBuf& parts, int32_t layer, const void* q, float sm_scale,
                          float* out, float* lse, hipStream_t stream, int32_t n_layers = 1,
                          int64_t layer_rows = 0, bool no_scratch = false) {
  const pkv::Shape& sh = p->core.shape();
  if (n_layers > 1 && plan.direct.empty()) {
    // the plan's launches once per layer (partial states reused in stream order)
    for (int32_t l = 0; l < n_layers; ++l) {
      const size_t rows = static_cast<size_t>(layer_rows) * l;
      pkv_status s = launch_plan(p, plan, lay, buf, parts, layer + l,
                                 static_cast<const uint16_t*>(q) + rows * sh.head_dim, sm_scale,
                                 out + rows * sh.head_dim, lse ? lse + rows : nullptr, stream, 1, 0,
                                 no_scratch);
      if (s != PKV_OK) return s;
    }
    return PKV_OK;
  }
  const char* base = static_cast<const char*>(buf.ptr);
  pkv_status s = ensure(p, parts, partial_bytes(plan, sh), stream);
  if (s != PKV_OK) return s;
  float* part_o = static_cast<float*>(parts.ptr);
  float* part_lse = part_o + static_cast<size_t>(plan.partial_rows) * sh.head_dim;

  if (plan.stride_mfma > pkv::kMaxItemBlocks || plan.stride_valu > pkv::kMaxItemBlocks ||
      plan.stride_direct > pkv::kMaxItemBlocks)
    return fail(PKV_ERR_ARG, "attention: a work item spans more blocks than the kernels stage");
  pkv::AttnParams ap{};
  ap.items = reinterpret_cast<const pkv::WorkItem*>(base + lay.items);
  ap.groups = reinterpret_cast<const pkv::RowGroup*>(base + lay.groups);
  ap.blocks = reinterpret_cast<const int32_t*>(base + lay.blocks);
  ap.q = static_cast<const uint16_t*>(q);
  ap.k_pool = p->k_pool;
  ap.v_pool = p->v_pool;
  ap.out = out;
  ap.lse = lse;
  ap.part_o = part_o;
  ap.part_lse = part_lse;
  ap.n_mfma = static_cast<int32_t>(plan.mfma.size());
  ap.stride_mfma = plan.stride_mfma;
  ap.stride_valu = plan.stride_valu;
  ap.layer = layer;
  ap.N = sh.num_blocks;
  ap.Hq = sh.num_q_heads;
  ap.Hkv = sh.num_kv_heads;
  ap.G = sh.num_q_heads / sh.num_kv_heads;
  ap.g_magic = static_cast<uint32_t>((65536 + ap.G - 1) / ap.G);
  ap.B = sh.block_size;
  ap.log2B = p->core.log2_block();
  ap.scale_log2 = sm_scale * pkv::kLog2eHost;
  const int32_t n_items = static_cast<int32_t>(plan.mfma.size() + plan.valu.size());
  hipEvent_t ev_a = nullptr, ev_b = nullptr;
  const bool timed = p->timing && (p->timing_tick++ % p->timing_every) == 0;
  if (timed) {
    s = take_event(p, &ev_a);
    if (s == PKV_OK) s = take_event(p, &ev_b);
    if (s != PKV_OK) return s;
  }
  // the events ride on the kernel's own dispatch: they take its start and end
  if (plan.tree) {
    // the MFMA items (if any) write their partial states, then the path
    // items merge them and write out / lse: events on the first launch's
    // start and the last one's end
    ap.steps = reinterpret_cast<const pkv::PathStep*>(base + lay.steps);
    ap.merges = reinterpret_cast<const pkv::MergeRow*>(base + lay.merges);
    const auto* paths = reinterpret_cast<const pkv::PathItem*>(base + lay.paths);
    const hipEvent_t ev_first = ev_a;
    if (!plan.mfma.empty()) {
      int32_t max_rows = 0;
      for (const pkv::WorkItem& it : plan.mfma) max_rows = std::max(max_rows, it.n_grp * ap.G);
      PKV_HIP(pkv::launch_wide(ap, static_cast<int32_t>(plan.mfma.size()), sh.head_dim, plan.stride_mfma,
                               max_rows, stream, ev_a, nullptr, no_scratch));
      ev_a = nullptr;
    }
    PKV_HIP(pkv::launch_path(ap, paths, static_cast<int32_t>(plan.paths.size()), sh.head_dim, stream, ev_a,
                             ev_b));
    if (timed) p->ev_pending.emplace_back(ev_first, ev_b);
    return PKV_OK;
  }
  // dense tiles only: the dense-tile kernel at head_dim 128; at head_dim 64
  // the mixed kernel (which also takes 256-row items as eight waves of two
  // tiles) measured faster (causal prefill of 4096 queries: 38.7 against
  // 44.2 us per launch)
  const bool dense_kernel = sh.head_dim == 128 || (plan.mfma_waves == 8 && plan.mfma_row_tiles != 2);
  if (plan.direct.empty() && plan.valu.empty() && !p->cfg.mixed_kernel_only && dense_kernel)
  {
    int32_t max_rows = 0;
    for (const pkv::WorkItem& it : plan.mfma) max_rows = std::max(max_rows, it.n_grp * ap.G);
    PKV_HIP(pkv::launch_wide(ap, n_items, sh.head_dim, plan.stride_mfma, max_rows, stream, ev_a, ev_b, no_scratch));
  }
  else if (plan.direct.empty())
    PKV_HIP(pkv::launch_attn(ap, n_items, sh.head_dim, plan.mfma_row_tiles,
                              plan.valu_max_rows * ap.G, plan.mfma_waves, stream, ev_a, ev_b));
  else {
    int32_t max_tok = 0;
    for (const pkv::WorkItem& it : plan.direct) max_tok = std::max(max_tok, it.n_tok);
    ap.layer_chunks = static_cast<uint64_t>(sh.num_blocks) * sh.num_kv_heads * sh.block_size * sh.head_dim / 8;
    ap.layer_rows = static_cast<uint64_t>(layer_rows);
    PKV_HIP(pkv::launch_direct(ap, static_cast<int32_t>(plan.direct.size()), sh.head_dim,
                                plan.stride_direct, max_tok, stream, ev_a, ev_b, n_layers));
  }
  if (timed) p->ev_pending.emplace_back(ev_a, ev_b);
  if (!plan.merges.empty()) {
    pkv::MergeParams mp{};
    mp.merges = reinterpret_cast<const pkv::MergeRow*>(base + lay.merges);
    mp.parts = reinterpret_cast<const int32_t*>(base + lay.parts);
    mp.part_o = part_o;
    mp.part_lse = part_lse;
    mp.out = out;
    mp.lse = lse;
    mp.Hq = sh.num_q_heads;
    mp.D = sh.head_dim;
    PKV_HIP(pkv::launch_merge(mp, static_cast<int32_t>(plan.merges.size()), stream));
  }
  return PKV_OK;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; }

// Planner knobs may be overridden from the environment for tuning sweeps:
// PKV_MFMA_MIN_ROWS (0 turns the MFMA kernel off), PKV_MFMA_ROW_TILES (1|2),
// PKV_MFMA_WAVES (4|8), PKV_UNSHARE_MAX_QUERIES, PKV_UNSHARE_MAX_TOKENS,
// PKV_TARGET_WGS, PKV_TARGET_MFMA_WGS, PKV_MAX_CHUNK, PKV_MAX_PARTS, PKV_WIDE_PAIRS,
// PKV_WIDE_MAX_PARTS, PKV_DIRECT_MAX_TOKENS
// and PKV_DIRECT_MAX_WGS (either 0 turns direct decode plans off), and
// PKV_MIXED_KERNEL_ONLY (1: plans of dense tiles only also run on the mixed
// MFMA / VALU kernel instead of the pipelined dense-tile kernel), and the
// tree decode planner's PKV_TREE_DECODE (0 turns it off), PKV_TREE_WIDE_ROWS,
// PKV_TREE_WIDE_TOKENS, PKV_TREE_PATH_TOKENS, PKV_TREE_ITEM_ROWS,
// PKV_TREE_TARGET_WGS, PKV_TREE_MAX_PARTS and PKV_TREE_MIN_WGS, and
// PKV_PRIVATE_SEGMENTS (1: every decode query one segment, no trie), and
// PKV_COARSE_PLANS (1: every call planned as the coarsest plan a workspace
// falls back to).
void apply_env(pkv::PlanConfig* c) {
  auto get = [](const char* name, int32_t* v, int32_t lo, int32_t hi) {
    const char* e = std::getenv(name);
    if (!e || !*e) return;
    long x = std::strtol(e, nullptr, 10);
    if (x >= lo && x <= hi) *v = static_cast<int32_t>(x);
  };
  get("PKV_MFMA_MIN_ROWS", &c->mfma_min_rows, 0, 1 << 20);
  get("PKV_MFMA_ROW_TILES", &c->mfma_row_tiles, 0, 2);
  get("PKV_MFMA_WAVES", &c->mfma_waves, 0, 8);
  get("PKV_UNSHARE_MAX_QUERIES", &c->unshare_max_queries, 0, 1 << 20);
  get("PKV_UNSHARE_MAX_TOKENS", &c->unshare_max_tokens, 0, 1 << 20);
  get("PKV_TARGET_WGS", &c->target_wgs, 1, 1 << 20);
  get("PKV_TARGET_MFMA_WGS", &c->target_mfma_wgs, 1, 1 << 20);
  get("PKV_MAX_CHUNK", &c->max_chunk, 64, 1 << 20);
  get("PKV_MAX_PARTS", &c->max_parts, 0, 1 << 20);
  get("PKV_WIDE_PAIRS", &c->wide_pairs, 0, 1 << 30);
  get("PKV_WIDE_MAX_PARTS", &c->wide_max_parts, 0, 1 << 20);
  get("PKV_DIRECT_MAX_TOKENS", &c->direct_max_tokens, 0, 1 << 20);
  get("PKV_DIRECT_MAX_WGS", &c->direct_max_wgs, 0, 1 << 30);
  get("PKV_MIXED_KERNEL_ONLY", &c->mixed_kernel_only, 0, 1);
  get("PKV_TREE_DECODE", &c->tree_decode, 0, 1);
  get("PKV_TREE_WIDE_ROWS", &c->tree_wide_rows, 1, 1 << 20);
  get("PKV_TREE_WIDE_TOKENS", &c->tree_wide_tokens, 1, 1 << 20);
  get("PKV_TREE_PATH_TOKENS", &c->tree_path_tokens, 1, 1 << 20);
  get("PKV_TREE_ITEM_ROWS", &c->tree_item_rows, 16, 256);
  get("PKV_TREE_TARGET_WGS", &c->tree_target_wgs, 1, 1 << 20);
  get("PKV_TREE_MAX_PARTS", &c->tree_max_parts, 1, pkv::kPathMaxParts);
  get("PKV_TREE_MIN_WGS", &c->tree_min_wgs, 0, 1 << 20);
  get("PKV_PRIVATE_SEGMENTS", &c->private_segments, 0, 1);
  int32_t coarse = 0;
  get("PKV_COARSE_PLANS", &coarse, 0, 1);
  if (coarse) *c = coarse_config(*c);
}

}  // namespace

extern "C" {

size_t kv_pool_bytes(const pkv_desc* d) {
  if (!d) return 0;
  pkv::Shape s{d->num_blocks, d->block_size, d->num_layers, d->num_q_heads, d->num_kv_heads, d->head_dim};
  if (!pkv::valid_shape(s, nullptr)) return 0;
  return static_cast<size_t>(s.num_layers) * s.num_blocks * s.num_kv_heads * s.block_size *
         s.head_dim * sizeof(uint16_t);
}

size_t kv_workspace_bytes(const pkv_desc* d, int32_t max_seqs, int32_t max_tree_nodes) {
  size_t r[4];
  return kv_workspace_layout(d, max_seqs, max_tree_nodes, r) == PKV_OK ? r[0] + r[1] + r[2] + r[3] : 0;
}

pkv_status kv_workspace_layout(const pkv_desc* d, int32_t max_seqs, int32_t max_tree_nodes, size_t* regions) {
  if (!d || !regions || max_seqs < 1 || max_seqs > 65536 || max_tree_nodes < 1 || max_tree_nodes > 65536)
    return fail(PKV_ERR_ARG, "kv_workspace_layout: NULL argument or limits outside 1 .. 65536");
  pkv::Shape s{d->num_blocks, d->block_size, d->num_layers, d->num_q_heads, d->num_kv_heads, d->head_dim};
  std::string why;
  if (!pkv::valid_shape(s, &why)) return fail(PKV_ERR_ARG, "kv_workspace_layout: " + why);
  const WsLayout w = ws_layout(s, max_seqs, max_tree_nodes);
  regions[0] = w.decode;
  regions[1] = w.verify;
  regions[2] = w.prefill;
  regions[3] = w.partials;
  return PKV_OK;
}

pkv_status kv_pool_create(const pkv_desc* d, void* k_pool, void* v_pool, const pkv_workspace* ws,
                          const int32_t* free_order, pkv_pool** out) {
  if (!d || !out) return fail(PKV_ERR_ARG, "kv_pool_create: desc and out must not be NULL");
  *out = nullptr;
  pkv::Shape s{d->num_blocks, d->block_size, d->num_layers, d->num_q_heads, d->num_kv_heads, d->head_dim};
  std::string why;
  if (!pkv::valid_shape(s, &why)) return fail(PKV_ERR_ARG, "kv_pool_create: " + why);
  if ((k_pool == nullptr) != (v_pool == nullptr))
    return fail(PKV_ERR_ARG, "kv_pool_create: give both device pools or neither");
  const bool device = k_pool != nullptr;
  if (device) {
    if (s.head_dim != 64 && s.head_dim != 128)
      return fail(PKV_ERR_UNSUPPORTED, "kv_pool_create: device pools need head_dim 64 or 128");
    if (s.num_q_heads / s.num_kv_heads > 16)
      return fail(PKV_ERR_UNSUPPORTED, "kv_pool_create: more than 16 query heads per kv head");
    if (!aligned16(k_pool) || !aligned16(v_pool))
      return fail(PKV_ERR_ARG, "kv_pool_create: pools must be 16-byte aligned");
    // the kernels address one layer of a pool in 32-bit units of 16 bytes
    const int64_t layer_chunks = static_cast<int64_t>(s.num_blocks) * s.num_kv_heads * s.block_size * s.head_dim / 8;
    if (layer_chunks >= (int64_t{1} << 32) || static_cast<int64_t>(s.num_kv_heads) * s.block_size * s.head_dim / 8 >= (1 << 24))
      return fail(PKV_ERR_UNSUPPORTED, "kv_pool_create: one layer of a device pool must stay under 64 GiB");
    // block ids enter the kernels' 24-bit multiplies
    if (s.num_blocks >= (1 << 24))
      return fail(PKV_ERR_UNSUPPORTED, "kv_pool_create: a device pool holds fewer than 2^24 blocks");
  }
  const pkv_workspace wsd = ws ? *ws : pkv_workspace{nullptr, 0, 0, 0};
  const int32_t max_seqs = wsd.max_seqs > 0 ? wsd.max_seqs : kDefaultMaxSeqs;
  const int32_t max_nodes = wsd.max_tree_nodes > 0 ? wsd.max_tree_nodes : kDefaultMaxNodes;
  if (wsd.max_seqs < 0 || wsd.max_tree_nodes < 0 || max_seqs > 65536 || max_nodes > 65536)
    return fail(PKV_ERR_ARG, "kv_pool_create: workspace limits must be 0 or 1 .. 65536");
  WsLayout wl;
  if (wsd.ptr) {
    if (!device) return fail(PKV_ERR_ARG, "kv_pool_create: a host-only pool takes no workspace");
    if ((reinterpret_cast<uintptr_t>(wsd.ptr) & (kWsAlign - 1)) != 0)
      return fail(PKV_ERR_ARG, "kv_pool_create: the workspace must be 256-byte aligned");
    wl = ws_layout(s, max_seqs, max_nodes);
    if (wsd.bytes < wl.total)
      return fail(PKV_ERR_ARG, "kv_pool_create: the workspace holds " + std::to_string(wsd.bytes) +
                                   " bytes, calls within its limits need " + std::to_string(wl.total));
  }
  if (free_order) {
    std::vector<char> seen(s.num_blocks, 0);
    for (int32_t i = 0; i < s.num_blocks; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= s.num_blocks || seen[b])
        return fail(PKV_ERR_ARG, "kv_pool_create: free_order is not a permutation of the block ids");
      seen[b] = 1;
    }
  }
  pkv_pool* p = new (std::nothrow) pkv_pool(s, free_order);
  if (!p) return fail(PKV_ERR_ARG, "kv_pool_create: out of host memory");
  p->device = device;
  apply_env(&p->cfg);
  if (device) {
    hipError_t e = hipGetDevice(&p->dev);
    if (e != hipSuccess) {
      delete p;
      return fail(PKV_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    }
    p->k_pool = static_cast<uint16_t*>(k_pool);
    p->v_pool = static_cast<uint16_t*>(v_pool);
    if (wsd.ptr) {
      // fixed regions of the caller's workspace, and pinned staging large
      // enough for any work list they hold, so calls allocate nothing
      p->ws_fixed = true;
      p->ws_max_seqs = max_seqs;
      p->ws_max_nodes = max_nodes;
      char* base = static_cast<char*>(wsd.ptr);
      size_t at = 0;
      for (auto [buf, bytes] : {std::pair<DevBuf*, size_t>{&p->decode_plan, wl.decode}, {&p->verify_plan, wl.verify},
                                {&p->prefill_plan, wl.prefill}, {&p->partials, wl.partials}}) {
        buf->ptr = base + at;
        buf->cap = bytes;
        buf->owned = false;
        at += bytes;
      }
      const size_t stage = std::max({wl.decode, wl.verify, wl.prefill});
      for (int i = 0; i < kStageSlots && e == hipSuccess; ++i) {
        e = hipHostMalloc(&p->stage[i], stage, hipHostMallocDefault);
        if (e == hipSuccess) p->stage_cap[i] = stage;
        else p->stage[i] = nullptr;
      }
      if (e != hipSuccess) {
        kv_pool_destroy(p);
        return fail(PKV_ERR_HIP, std::string("kv_pool_create: pinned staging: ") + hipGetErrorString(e));
      }
    }
  }
  *out = p;
  return PKV_OK;
}

size_t kv_pool_q4_bytes(const pkv_desc* d, size_t* norm_bytes) {
  if (norm_bytes) *norm_bytes = 0;
  if (!d) return 0;
  pkv::Shape s{d->num_blocks, d->block_size, d->num_layers, d->num_q_heads, d->num_kv_heads, d->head_dim};
  if (!pkv::valid_shape(s, nullptr)) return 0;
  const size_t vecs = static_cast<size_t>(s.num_layers) * s.num_blocks * s.num_kv_heads * s.block_size;
  if (norm_bytes) *norm_bytes = vecs * sizeof(uint16_t);
  return vecs * static_cast<size_t>(s.head_dim / 2);
}

pkv_status kv_pool_create_q4(const pkv_desc* d, void* k_codes, void* v_codes, void* k_norms,
                             void* v_norms, const int8_t* signs, const int32_t* free_order,
                             pkv_pool** out) {
  if (!d || !out) return fail(PKV_ERR_ARG, "kv_pool_create_q4: desc and out must not be NULL");
  *out = nullptr;
  if (!k_codes || !v_codes || !k_norms || !v_norms || !signs)
    return fail(PKV_ERR_ARG, "kv_pool_create_q4: codes, norms and signs are required");
  if (!aligned16(k_codes) || !aligned16(v_codes) || !aligned16(k_norms) || !aligned16(v_norms))
    return fail(PKV_ERR_ARG, "kv_pool_create_q4: device arrays must be 16-byte aligned");
  pkv::Shape s{d->num_blocks, d->block_size, d->num_layers, d->num_q_heads, d->num_kv_heads, d->head_dim};
  std::string why;
  if (!pkv::valid_shape(s, &why)) return fail(PKV_ERR_ARG, "kv_pool_create_q4: " + why);
  if (s.head_dim != 64 && s.head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "kv_pool_create_q4: head_dim must be 64 or 128");
  for (int32_t i = 0; i < s.head_dim; ++i)
    if (signs[i] != 1 && signs[i] != -1) return fail(PKV_ERR_ARG, "kv_pool_create_q4: signs must be +1 or -1");
  // a placeholder bf16 pair keeps the device path of kv_pool_create; never read
  pkv_status st = kv_pool_create(d, k_codes, v_codes, nullptr, free_order, out);
  if (st != PKV_OK) return st;
  pkv_pool* p = *out;
  p->q4 = true;
  p->k_pool = p->v_pool = nullptr;
  p->k_codes = static_cast<uint8_t*>(k_codes);
  p->v_codes = static_cast<uint8_t*>(v_codes);
  p->k_norms = static_cast<uint16_t*>(k_norms);
  p->v_norms = static_cast<uint16_t*>(v_norms);
  std::vector<float> sf(signs, signs + s.head_dim);
  for (float& f : sf) f = f > 0 ? 1.f : -1.f;
  DeviceGuard g(p->dev);
  hipError_t e = hipMalloc(&p->signs.ptr, sf.size() * sizeof(float));
  if (e == hipSuccess) {
    p->signs.cap = sf.size() * sizeof(float);
    e = hipMemcpy(p->signs.ptr, sf.data(), sf.size() * sizeof(float), hipMemcpyHostToDevice);
  }
  if (e != hipSuccess) {
    kv_pool_destroy(p);
    *out = nullptr;
    return fail(PKV_ERR_HIP, std::string("kv_pool_create_q4: ") + hipGetErrorString(e));
  }
  return PKV_OK;
}

void kv_pool_destroy(pkv_pool* p) {
  if (!p) return;
  detach_radixes(p);
  if (p->device) {
    DeviceGuard g(p->dev);
    (void)hipDeviceSynchronize();
    for (DevBuf* b : {&p->append_plan, &p->commit_plan, &p->decode_plan, &p->verify_plan, &p->prefill_plan, &p->partials, &p->signs})
      if (b->ptr && b->owned) (void)hipFree(b->ptr);
    for (auto& r : p->retired) {
      (void)hipFree(r.first);
      (void)hipEventDestroy(r.second);
    }
    for (int i = 0; i < kStageSlots; ++i) {
      if (p->stage[i]) (void)hipHostFree(p->stage[i]);
      if (p->stage_ev[i]) (void)hipEventDestroy(p->stage_ev[i]);
    }
    for (hipEvent_t e : p->ev_free) (void)hipEventDestroy(e);
    for (auto& pr : p->ev_pending) {
      (void)hipEventDestroy(pr.first);
      (void)hipEventDestroy(pr.second);
    }
  }
  delete p;
}

pkv_status seq_allocate(pkv_pool* p, int64_t* out_seq) {
  if (!p || !out_seq) return fail(PKV_ERR_ARG, "seq_allocate: NULL argument");
  *out_seq = p->core.allocate();
  return PKV_OK;
}

pkv_status seq_fork(pkv_pool* p, int64_t parent, int64_t* out_child) {
  if (!p || !out_child) return fail(PKV_ERR_ARG, "seq_fork: NULL argument");
  std::string why;
  pkv::Err e = p->core.fork(parent, out_child, &why);
  return e == pkv::Err::ok ? PKV_OK : fail(to_status(e), why);
}

pkv_status seq_free(pkv_pool* p, int64_t seq) {
  if (!p) return fail(PKV_ERR_ARG, "seq_free: NULL pool");
  std::string why;
  pkv::Err e = p->core.release(seq, &why);
  return e == pkv::Err::ok ? PKV_OK : fail(to_status(e), why);
}

pkv_status kv_append(pkv_pool* p, const int64_t* seqs, int32_t n_seqs, int32_t n_tok,
                     const void* k_new, const void* v_new, void* stream) {
  if (!p) return fail(PKV_ERR_ARG, "kv_append: NULL pool");
  const bool has_work = n_seqs > 0 && n_tok > 0;
  if (p->device) {
    if (has_work && (!k_new || !v_new))
      return fail(PKV_ERR_ARG, "kv_append: k_new and v_new are required for a device pool");
    if (has_work && (!aligned16(k_new) || !aligned16(v_new)))
      return fail(PKV_ERR_ARG, "kv_append: k_new / v_new must be 16-byte aligned");
  } else if (k_new || v_new) {
    return fail(PKV_ERR_ARG, "kv_append: a host-only pool takes no K/V data");
  }
  pkv::PendingAppend pa;
  std::string why;
  pkv::Err e = p->core.prepare_append(seqs, n_seqs, n_tok, &pa, &why);
  if (e != pkv::Err::ok) return fail(to_status(e), why);
  if (p->device && has_work) {
    DeviceGuard g(p->dev);
    PKV_HIP(g.err);
    const pkv::Shape& sh = p->core.shape();
    hipStream_t st = static_cast<hipStream_t>(stream);
    const size_t slot_bytes = pa.result.slots.size() * sizeof(int32_t);
    const size_t cow_off = align16(slot_bytes);
    const size_t bytes = cow_off + pa.result.cow.size() * 3 * sizeof(int32_t);
    pkv_status s = upload(p, p->append_plan, bytes, st, [&](char* dst) {
      std::memcpy(dst, pa.result.slots.data(), slot_bytes);
      int32_t* c = reinterpret_cast<int32_t*>(dst + cow_off);
      for (size_t k = 0; k < pa.result.cow.size(); ++k) {
        c[3 * k + 0] = pa.result.cow[k].src;
        c[3 * k + 1] = pa.result.cow[k].dst;
        c[3 * k + 2] = pa.result.cow[k].n_slots;
      }
    });
    if (s != PKV_OK) return s;
    if (p->q4) {
      pkv::Q4AppendParams qp{};
      qp.k_new = static_cast<const uint16_t*>(k_new);
      qp.v_new = static_cast<const uint16_t*>(v_new);
      qp.k_codes = p->k_codes;
      qp.v_codes = p->v_codes;
      qp.k_norms = p->k_norms;
      qp.v_norms = p->v_norms;
      qp.signs = static_cast<const float*>(p->signs.ptr);
      qp.slots = static_cast<const int32_t*>(p->append_plan.ptr);
      qp.cow = reinterpret_cast<const int32_t*>(static_cast<const char*>(p->append_plan.ptr) + cow_off);
      qp.n_rows = n_seqs * n_tok;
      qp.n_cow = static_cast<int32_t>(pa.result.cow.size());
      qp.L = sh.num_layers;
      qp.N = sh.num_blocks;
      qp.Hkv = sh.num_kv_heads;
      qp.B = sh.block_size;
      qp.log2B = p->core.log2_block();
      qp.D = sh.head_dim;
      PKV_HIP(pkv::launch_q4_append(qp, st));
      p->core.commit_append(std::move(pa));
      return PKV_OK;
    }
    pkv::AppendParams ap{};
    ap.k_new = static_cast<const uint16_t*>(k_new);
    ap.v_new = static_cast<const uint16_t*>(v_new);
    ap.k_pool = p->k_pool;
    ap.v_pool = p->v_pool;
    ap.slots = static_cast<const int32_t*>(p->append_plan.ptr);
    ap.cow = reinterpret_cast<const int32_t*>(static_cast<const char*>(p->append_plan.ptr) + cow_off);
    ap.n_rows = n_seqs * n_tok;
    ap.n_cow = static_cast<int32_t>(pa.result.cow.size());
    ap.L = sh.num_layers;
    ap.N = sh.num_blocks;
    ap.Hkv = sh.num_kv_heads;
    ap.B = sh.block_size;
    ap.log2B = p->core.log2_block();
    ap.D = sh.head_dim;
    PKV_HIP(pkv::launch_append(ap, st));
  }
  p->core.commit_append(std::move(pa));
  return PKV_OK;
}

pkv_status kv_tree_commit(pkv_pool* p, const int64_t* seqs, int32_t n_seqs, int32_t n_nodes,
                          const int32_t* parent, const int32_t* path_len, const int32_t* paths,
                          void* stream) {
  if (!p) return fail(PKV_ERR_ARG, "kv_tree_commit: NULL pool");
  if (p->q4) return fail(PKV_ERR_UNSUPPORTED, "kv_tree_commit: 4-bit pools support decode only");
  if (n_seqs == 0) return PKV_OK;
  // the commit launch takes one grid row per sequence (checked before any
  // work is enqueued)
  if (n_seqs > 65535) return fail(PKV_ERR_ARG, "kv_tree_commit: at most 65535 sequences per call");
  pkv::PendingCommit pc;
  std::string why;
  pkv::Err e = p->core.prepare_commit(seqs, n_seqs, n_nodes, parent, path_len, paths, &pc, &why);
  if (e != pkv::Err::ok) return fail(to_status(e), why);
  if (p->device && (!pc.cow.empty() || !pc.move_src.empty())) {
    DeviceGuard g(p->dev);
    PKV_HIP(g.err);
    const pkv::Shape& sh = p->core.shape();
    hipStream_t st = static_cast<hipStream_t>(stream);
    const size_t n_mv = pc.move_src.size();
    const size_t off_src = align16((pc.seq_cow.size() + pc.seq_move.size()) * sizeof(int32_t));
    const size_t off_dst = off_src + align16(n_mv * sizeof(int32_t));
    const size_t off_cow = off_dst + align16(n_mv * sizeof(int32_t));
    const size_t bytes = off_cow + pc.cow.size() * 3 * sizeof(int32_t);
    pkv_status s = upload(p, p->commit_plan, bytes, st, [&](char* dst) {
      std::memcpy(dst, pc.seq_cow.data(), pc.seq_cow.size() * sizeof(int32_t));
      std::memcpy(dst + pc.seq_cow.size() * sizeof(int32_t), pc.seq_move.data(),
                  pc.seq_move.size() * sizeof(int32_t));
      std::memcpy(dst + off_src, pc.move_src.data(), n_mv * sizeof(int32_t));
      std::memcpy(dst + off_dst, pc.move_dst.data(), n_mv * sizeof(int32_t));
      int32_t* c = reinterpret_cast<int32_t*>(dst + off_cow);
      for (size_t k = 0; k < pc.cow.size(); ++k) {
        c[3 * k + 0] = pc.cow[k].src;
        c[3 * k + 1] = pc.cow[k].dst;
        c[3 * k + 2] = pc.cow[k].n_slots;
      }
    });
    if (s != PKV_OK) return s;
    const char* base = static_cast<const char*>(p->commit_plan.ptr);
    pkv::CommitParams cp{};
    cp.k_pool = p->k_pool;
    cp.v_pool = p->v_pool;
    cp.seq_cow = reinterpret_cast<const int32_t*>(base);
    cp.seq_move = cp.seq_cow + pc.seq_cow.size();
    cp.move_src = reinterpret_cast<const int32_t*>(base + off_src);
    cp.move_dst = reinterpret_cast<const int32_t*>(base + off_dst);
    cp.cow = reinterpret_cast<const int32_t*>(base + off_cow);
    cp.L = sh.num_layers;
    cp.N = sh.num_blocks;
    cp.Hkv = sh.num_kv_heads;
    cp.B = sh.block_size;
    cp.log2B = p->core.log2_block();
    cp.D = sh.head_dim;
    if (!pc.conflict) {
      cp.seq0 = 0;
      PKV_HIP(pkv::launch_commit(cp, n_seqs, st));
    } else {
      // a block written in place by one sequence is read by another: in order
      for (int32_t i = 0; i < n_seqs; ++i) {
        cp.seq0 = i;
        PKV_HIP(pkv::launch_commit(cp, 1, st));
      }
    }
  }
  p->core.commit_commit(std::move(pc));
  return PKV_OK;
}

namespace {

// Decode over a 4-bit pool: one workgroup per (query, kv head) over all of
// the query's keys, straight from the codes.
pkv_status decode_q4(pkv_pool* p, int32_t layer, const int64_t* seqs, int32_t n_seqs, const void* q,
                     float sm_scale, float* out, float* lse, void* stream) {
  const pkv::Shape& sh = p->core.shape();
  p->q4_items.clear();
  p->q4_blocks.clear();
  for (int32_t i = 0; i < n_seqs; ++i) {
    const pkv::SeqState* st = p->core.find(seqs[i]);
    if (!st) return fail(PKV_ERR_SEQ, "paged_attn_decode: unknown sequence " + std::to_string(seqs[i]));
    if (st->len == 0) return fail(PKV_ERR_EMPTY, "paged_attn_decode: empty sequence " + std::to_string(seqs[i]));
    p->q4_items.push_back(pkv::Q4Item{static_cast<int32_t>(p->q4_blocks.size()), st->len, i, 0});
    p->q4_blocks.insert(p->q4_blocks.end(), st->table.begin(), st->table.end());
  }
  DeviceGuard g(p->dev);
  PKV_HIP(g.err);
  hipStream_t stv = static_cast<hipStream_t>(stream);
  const size_t items_bytes = p->q4_items.size() * sizeof(pkv::Q4Item);
  const size_t blk_off = align16(items_bytes);
  const size_t bytes = blk_off + p->q4_blocks.size() * sizeof(int32_t);
  pkv_status s = upload(p, p->decode_plan, bytes, stv, [&](char* dst) {
    std::memcpy(dst, p->q4_items.data(), items_bytes);
    std::memcpy(dst + blk_off, p->q4_blocks.data(), p->q4_blocks.size() * sizeof(int32_t));
  });
  if (s != PKV_OK) return s;
  p->dcache_valid = false;   // the decode plan buffer now holds this call's lists
  const char* base = static_cast<const char*>(p->decode_plan.ptr);
  pkv::Q4DecodeParams dp{};
  dp.items = reinterpret_cast<const pkv::Q4Item*>(base);
  dp.blocks = reinterpret_cast<const int32_t*>(base + blk_off);
  dp.q = static_cast<const uint16_t*>(q);
  dp.k_codes = p->k_codes;
  dp.v_codes = p->v_codes;
  dp.k_norms = p->k_norms;
  dp.v_norms = p->v_norms;
  dp.signs = static_cast<const float*>(p->signs.ptr);
  dp.out = out;
  dp.lse = lse;
  dp.layer = layer;
  dp.N = sh.num_blocks;
  dp.Hq = sh.num_q_heads;
  dp.Hkv = sh.num_kv_heads;
  dp.G = sh.num_q_heads / sh.num_kv_heads;
  dp.B = sh.block_size;
  dp.log2B = p->core.log2_block();
  dp.scale_log2 = sm_scale * pkv::kLog2eHost;
  hipEvent_t ev_a = nullptr, ev_b = nullptr;
  const bool timed = p->timing && (p->timing_tick++ % p->timing_every) == 0;
  if (timed) {
    s = take_event(p, &ev_a);
    if (s == PKV_OK) s = take_event(p, &ev_b);
    if (s != PKV_OK) return s;
  }
  PKV_HIP(pkv::launch_q4_decode(dp, n_seqs, sh.head_dim, stv, ev_a, ev_b));
  if (timed) p->ev_pending.emplace_back(ev_a, ev_b);
  return PKV_OK;
}

}  // namespace

}  // extern "C"

namespace {

// The decode plan of a call -- the cached one, patched, or made afresh and
// fitted to the workspace -- uploaded to the pool's decode region on `st`.
pkv_status decode_prepare(pkv_pool* p, const int64_t* seqs, int32_t n_seqs, hipStream_t st) {
  const bool same_seqs = p->dcache_valid && p->dcache_seqs.size() == static_cast<size_t>(n_seqs) &&
                         std::memcmp(p->dcache_seqs.data(), seqs, n_seqs * sizeof(int64_t)) == 0;
  bool hit = same_seqs && p->dcache_version == p->core.version();
  if (same_seqs && !hit && pkv::patch_decode(p->core, seqs, n_seqs, p->cfg, &p->dplan)) {
    // appends only filled the sequences' last blocks: same plan, longer tail items
    if (!plan_fits_kernels(p->dplan, p->core.shape())) {
      p->dcache_valid = false;
      return fail(PKV_ERR_ARG, "paged_attn_decode: internal plan exceeds the kernels' tile limits");
    }
    pkv_status s = upload(p, p->decode_plan, p->dlayout.total, st,
                          [&](char* dst) { serialize(p->dplan, p->dlayout, dst); });
    if (s != PKV_OK) {
      p->dcache_valid = false;
      return s;
    }
    p->dcache_version = p->core.version();
    hit = true;
  }
  if (!hit) {
    p->dcache_valid = false;
    pkv_status s = plan_to_fit(p, p->decode_plan, p->partials, "paged_attn_decode", &p->dplan, &p->dlayout,
                               [&](const pkv::PlanConfig& c, pkv::Plan* pl, std::string* why) {
                                 return pkv::plan_decode(p->core, seqs, n_seqs, c, pl, why);
                               });
    if (s != PKV_OK) return s;
    if (!plan_fits_kernels(p->dplan, p->core.shape()))
      return fail(PKV_ERR_ARG, "paged_attn_decode: internal plan exceeds the kernels' tile limits");
    s = ensure(p, p->partials, partial_bytes(p->dplan, p->core.shape()), st);
    if (s != PKV_OK) return s;
    s = upload(p, p->decode_plan, p->dlayout.total, st,
                          [&](char* dst) { serialize(p->dplan, p->dlayout, dst); });
    if (s != PKV_OK) return s;
    p->dcache_seqs.assign(seqs, seqs + n_seqs);
    p->dcache_version = p->core.version();
    p->dcache_valid = true;
  }
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status paged_attn_decode(pkv_pool* p, int32_t layer, const int64_t* seqs, int32_t n_seqs,
                             const void* q, float sm_scale, float* out, float* lse, void* stream) {
  if (!p) return fail(PKV_ERR_ARG, "paged_attn_decode: NULL pool");
  if (!p->device) return fail(PKV_ERR_ARG, "paged_attn_decode: the pool has no device storage");
  if (n_seqs < 0) return fail(PKV_ERR_ARG, "paged_attn_decode: negative n_seqs");
  if (n_seqs == 0) return PKV_OK;
  if (!seqs || !q || !out) return fail(PKV_ERR_ARG, "paged_attn_decode: NULL seqs, q or out");
  if (layer < 0 || layer >= p->core.shape().num_layers)
    return fail(PKV_ERR_ARG, "paged_attn_decode: layer out of range");
  if (!aligned16(q) || !aligned16(out))
    return fail(PKV_ERR_ARG, "paged_attn_decode: q and out must be 16-byte aligned");
  if (p->ws_fixed && n_seqs > p->ws_max_seqs)
    return fail(PKV_ERR_ARG, "paged_attn_decode: more sequences than the workspace's max_seqs");
  if (p->q4) return decode_q4(p, layer, seqs, n_seqs, q, sm_scale, out, lse, stream);
  DeviceGuard g(p->dev);
  PKV_HIP(g.err);
  hipStream_t st = static_cast<hipStream_t>(stream);
  pkv_status s = decode_prepare(p, seqs, n_seqs, st);
  if (s != PKV_OK) return s;
  return launch_plan(p, p->dplan, p->dlayout, p->decode_plan, p->partials, layer, q, sm_scale, out, lse, st);
}

pkv_status paged_attn_decode_layers(pkv_pool* p, int32_t layer0, int32_t n_layers, const int64_t* seqs,
                                    int32_t n_seqs, const void* q, float sm_scale, float* out, float* lse,
                                    void* stream) {
  if (!p) return fail(PKV_ERR_ARG, "paged_attn_decode_layers: NULL pool");
  if (!p->device) return fail(PKV_ERR_ARG, "paged_attn_decode_layers: the pool has no device storage");
  if (p->q4) return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode_layers: 4-bit pools are not supported");
  if (n_seqs < 0) return fail(PKV_ERR_ARG, "paged_attn_decode_layers: negative n_seqs");
  if (layer0 < 0 || n_layers < 1 || n_layers > 65535 ||
      static_cast<int64_t>(layer0) + n_layers > p->core.shape().num_layers)
    return fail(PKV_ERR_ARG, "paged_attn_decode_layers: layer range outside the pool's layers");
  if (n_seqs == 0) return PKV_OK;
  if (!seqs || !q || !out) return fail(PKV_ERR_ARG, "paged_attn_decode_layers: NULL seqs, q or out");
  if (!aligned16(q) || !aligned16(out))
    return fail(PKV_ERR_ARG, "paged_attn_decode_layers: q and out must be 16-byte aligned");
  if (p->ws_fixed && n_seqs > p->ws_max_seqs)
    return fail(PKV_ERR_ARG, "paged_attn_decode_layers: more sequences than the workspace's max_seqs");
  DeviceGuard g(p->dev);
  PKV_HIP(g.err);
  hipStream_t st = static_cast<hipStream_t>(stream);
  pkv_status s = decode_prepare(p, seqs, n_seqs, st);
  if (s != PKV_OK) return s;
  return launch_plan(p, p->dplan, p->dlayout, p->decode_plan, p->partials, layer0, q, sm_scale, out, lse, st,
                     n_layers, static_cast<int64_t>(n_seqs) * p->core.shape().num_q_heads);
}

}  // extern "C"

// ---- decode without allocation -------------------------------------------
//
// paged_attn_decode_scratch keeps its work lists and partial states in one
// file-scope device array instead of the pool's buffers.  In host code the
// array's name stands for no device address: each device's copy is looked
// up once (hipGetSymbolAddress, with that device current) and only that
// address is handed to copies and kernels.
namespace {

constexpr size_t kScratchBytes = size_t{32} << 20;
constexpr size_t kScratchPlanBytes = size_t{8} << 20;   // work lists; the rest holds partial states
constexpr int kScratchDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
char* g_scratch_addr[kScratchDevices] = {};

// The address of `dev`'s copy of scratch; `dev` must be the current device.
pkv_status scratch_address(int dev, char** out) {
  if (dev < 0 || dev >= kScratchDevices)
    return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode_scratch: device index past the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(PKV_ERR_HIP, std::string("paged_attn_decode_scratch: hipGetSymbolAddress: ") +
                                   hipGetErrorString(e));
    g_scratch_addr[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch_addr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status paged_attn_decode_scratch(pkv_pool* p, int32_t layer, const int64_t* seqs, int32_t n_seqs,
                                     const void* q, float sm_scale, float* out, float* lse, void* stream) {
  if (!p) return fail(PKV_ERR_ARG, "paged_attn_decode_scratch: NULL pool");
  if (!p->device) return fail(PKV_ERR_ARG, "paged_attn_decode_scratch: the pool has no device storage");
  if (p->q4) return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode_scratch: 4-bit pools are not supported");
  if (n_seqs < 0) return fail(PKV_ERR_ARG, "paged_attn_decode_scratch: negative n_seqs");
  if (n_seqs == 0) return PKV_OK;
  if (!seqs || !q || !out) return fail(PKV_ERR_ARG, "paged_attn_decode_scratch: NULL seqs, q or out");
  if (layer < 0 || layer >= p->core.shape().num_layers)
    return fail(PKV_ERR_ARG, "paged_attn_decode_scratch: layer out of range");
  if (!aligned16(q) || !aligned16(out))
    return fail(PKV_ERR_ARG, "paged_attn_decode_scratch: q and out must be 16-byte aligned");
  DeviceGuard g(p->dev);
  PKV_HIP(g.err);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* base = nullptr;
  pkv_status s = scratch_address(p->dev, &base);
  if (s != PKV_OK) return s;
  DevBuf lists{base, kScratchPlanBytes, false};
  DevBuf parts{base + kScratchPlanBytes, kScratchBytes - kScratchPlanBytes, false};
  // planned afresh each call (the array may hold another pool's lists),
  // coarse when the pool's settings give more than the array holds
  s = plan_to_fit(p, lists, parts, "paged_attn_decode_scratch", &p->splan, &p->slayout,
                  [&](const pkv::PlanConfig& c, pkv::Plan* pl, std::string* why) {
                    return pkv::plan_decode(p->core, seqs, n_seqs, c, pl, why);
                  });
  if (s != PKV_OK) return s;
  if (!plan_fits_kernels(p->splan, p->core.shape()))
    return fail(PKV_ERR_ARG, "paged_attn_decode_scratch: internal plan exceeds the kernels' tile limits");
  // from pageable host memory: the runtime stages the copy itself
  p->sstage.resize(p->slayout.total);
  serialize(p->splan, p->slayout, p->sstage.data());
  if (p->slayout.total > 0)
    PKV_HIP(hipMemcpyAsync(lists.ptr, p->sstage.data(), p->slayout.total, hipMemcpyHostToDevice, st));
  return launch_plan(p, p->splan, p->slayout, lists, parts, layer, q, sm_scale, out, lse, st, 1, 0,
                     /*no_scratch=*/true);
}

pkv_status paged_attn_tree_verify(pkv_pool* p, int32_t layer, const int64_t* seqs, int32_t n_seqs,
                                  int32_t n_nodes, const int32_t* parent, const void* q,
                                  float sm_scale, float* out, float* lse, void* stream) {
  if (!p) return fail(PKV_ERR_ARG, "paged_attn_tree_verify: NULL pool");
  if (!p->device) return fail(PKV_ERR_ARG, "paged_attn_tree_verify: the pool has no device storage");
  if (p->q4) return fail(PKV_ERR_UNSUPPORTED, "paged_attn_tree_verify: 4-bit pools support decode only");
  if (n_seqs < 0) return fail(PKV_ERR_ARG, "paged_attn_tree_verify: negative n_seqs");
  if (n_seqs == 0) return PKV_OK;
  if (!seqs || !parent || !q || !out)
    return fail(PKV_ERR_ARG, "paged_attn_tree_verify: NULL seqs, parent, q or out");
  if (layer < 0 || layer >= p->core.shape().num_layers)
    return fail(PKV_ERR_ARG, "paged_attn_tree_verify: layer out of range");
  if (!aligned16(q) || !aligned16(out))
    return fail(PKV_ERR_ARG, "paged_attn_tree_verify: q and out must be 16-byte aligned");
  if (p->ws_fixed && (n_seqs > p->ws_max_seqs || n_nodes > p->ws_max_nodes))
    return fail(PKV_ERR_ARG, "paged_attn_tree_verify: more sequences or tree nodes than the workspace's limits");
  const size_t n_par = static_cast<size_t>(n_seqs) * (n_nodes > 0 ? n_nodes : 0);
  const bool hit = p->vcache_valid && p->vcache_version == p->core.version() && p->vcache_nodes == n_nodes &&
                   p->vcache_seqs.size() == static_cast<size_t>(n_seqs) &&
                   std::memcmp(p->vcache_seqs.data(), seqs, n_seqs * sizeof(int64_t)) == 0 &&
                   std::memcmp(p->vcache_parent.data(), parent, n_par * sizeof(int32_t)) == 0;
  DeviceGuard g(p->dev);
  PKV_HIP(g.err);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!hit) {
    p->vcache_valid = false;
    pkv_status s = plan_to_fit(p, p->verify_plan, p->partials, "paged_attn_tree_verify", &p->vplan, &p->vlayout,
                               [&](const pkv::PlanConfig& c, pkv::Plan* pl, std::string* why) {
                                 return pkv::plan_verify(p->core, seqs, n_seqs, n_nodes, parent, c, pl, why);
                               });
    if (s != PKV_OK) return s;
    if (!plan_fits_kernels(p->vplan, p->core.shape()))
      return fail(PKV_ERR_ARG, "paged_attn_tree_verify: internal plan exceeds the kernels' tile limits");
    s = ensure(p, p->partials, partial_bytes(p->vplan, p->core.shape()), st);
    if (s != PKV_OK) return s;
    s = upload(p, p->verify_plan, p->vlayout.total, st,
               [&](char* dst) { serialize(p->vplan, p->vlayout, dst); });
    if (s != PKV_OK) return s;
    p->vcache_seqs.assign(seqs, seqs + n_seqs);
    p->vcache_parent.assign(parent, parent + n_par);
    p->vcache_nodes = n_nodes;
    p->vcache_version = p->core.version();
    p->vcache_valid = true;
  }
  return launch_plan(p, p->vplan, p->vlayout, p->verify_plan, p->partials, layer, q, sm_scale, out, lse, st);
}

pkv_status paged_attn_prefill(pkv_pool* p, int32_t layer, const int64_t* seqs, int32_t n_seqs,
                              const int32_t* n_new, const void* q, float sm_scale, float* out,
                              float* lse, void* stream) {
  if (!p) return fail(PKV_ERR_ARG, "paged_attn_prefill: NULL pool");
  if (!p->device) return fail(PKV_ERR_ARG, "paged_attn_prefill: the pool has no device storage");
  if (p->q4) return fail(PKV_ERR_UNSUPPORTED, "paged_attn_prefill: 4-bit pools support decode only");
  if (n_seqs < 0) return fail(PKV_ERR_ARG, "paged_attn_prefill: negative n_seqs");
  if (n_seqs == 0) return PKV_OK;
  if (!seqs || !n_new) return fail(PKV_ERR_ARG, "paged_attn_prefill: NULL seqs or n_new");
  if (layer < 0 || layer >= p->core.shape().num_layers)
    return fail(PKV_ERR_ARG, "paged_attn_prefill: layer out of range");
  if (p->ws_fixed) {
    if (n_seqs > p->ws_max_seqs)
      return fail(PKV_ERR_ARG, "paged_attn_prefill: more sequences than the workspace's max_seqs");
    for (int32_t i = 0; i < n_seqs; ++i)
      if (n_new[i] > p->ws_max_nodes)
        return fail(PKV_ERR_ARG, "paged_attn_prefill: more new tokens than the workspace's max_tree_nodes");
  }
  const bool hit = p->pcache_valid && p->pcache_version == p->core.version() &&
                   p->pcache_seqs.size() == static_cast<size_t>(n_seqs) &&
                   std::memcmp(p->pcache_seqs.data(), seqs, n_seqs * sizeof(int64_t)) == 0 &&
                   std::memcmp(p->pcache_new.data(), n_new, n_seqs * sizeof(int32_t)) == 0;
  if (!hit) {
    p->pcache_valid = false;
    pkv_status s = plan_to_fit(p, p->prefill_plan, p->partials, "paged_attn_prefill", &p->pplan, &p->playout,
                               [&](const pkv::PlanConfig& c, pkv::Plan* pl, std::string* why) {
                                 return pkv::plan_prefill(p->core, seqs, n_seqs, n_new, c, pl, why);
                               });
    if (s != PKV_OK) return s;
  }
  if (p->pplan.mfma.empty() && p->pplan.valu.empty()) return PKV_OK;   // no new tokens
  if (!q || !out) return fail(PKV_ERR_ARG, "paged_attn_prefill: NULL q or out");
  if (!aligned16(q) || !aligned16(out))
    return fail(PKV_ERR_ARG, "paged_attn_prefill: q and out must be 16-byte aligned");
  DeviceGuard g(p->dev);
  PKV_HIP(g.err);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!hit) {
    if (!plan_fits_kernels(p->pplan, p->core.shape()))
      return fail(PKV_ERR_ARG, "paged_attn_prefill: internal plan exceeds the kernels' tile limits");
    pkv_status s = ensure(p, p->partials, partial_bytes(p->pplan, p->core.shape()), st);
    if (s != PKV_OK) return s;
    s = upload(p, p->prefill_plan, p->playout.total, st,
                          [&](char* dst) { serialize(p->pplan, p->playout, dst); });
    if (s != PKV_OK) return s;
    p->pcache_seqs.assign(seqs, seqs + n_seqs);
    p->pcache_new.assign(n_new, n_new + n_seqs);
    p->pcache_version = p->core.version();
    p->pcache_valid = true;
  }
  return launch_plan(p, p->pplan, p->playout, p->prefill_plan, p->partials, layer, q, sm_scale, out, lse, st);
}

// ---- radix prefix cache --------------------------------------------------

pkv_status radix_create(pkv_pool* p, pkv_radix** out) {
  if (!p || !out) return fail(PKV_ERR_ARG, "radix_create: NULL argument");
  *out = new (std::nothrow) pkv_radix(p);
  if (!*out) return fail(PKV_ERR_OOM, "radix_create: out of host memory");
  p->radixes.push_back(*out);
  return PKV_OK;
}

void radix_destroy(pkv_radix* r) {
  if (!r) return;
  if (r->pool) {
    auto& v = r->pool->radixes;
    v.erase(std::remove(v.begin(), v.end(), r), v.end());
  }
  delete r;
}

pkv_status radix_match(pkv_radix* r, const int32_t* tokens, int32_t n_tokens, int64_t* out_seq,
                       int32_t* out_matched) {
  if (!r || !out_seq || !out_matched) return fail(PKV_ERR_ARG, "radix_match: NULL argument");
  if (!r->pool) return fail(PKV_ERR_ARG, "radix_match: the cache's pool was destroyed");
  std::string why;
  pkv::Err e = r->cache.match(tokens, n_tokens, out_seq, out_matched, &why);
  return e == pkv::Err::ok ? PKV_OK : fail(to_status(e), why);
}

pkv_status radix_insert(pkv_radix* r, int64_t seq, const int32_t* tokens, int32_t n_tokens) {
  if (!r) return fail(PKV_ERR_ARG, "radix_insert: NULL cache");
  if (!r->pool) return fail(PKV_ERR_ARG, "radix_insert: the cache's pool was destroyed");
  std::string why;
  pkv::Err e = r->cache.insert(seq, tokens, n_tokens, &why);
  return e == pkv::Err::ok ? PKV_OK : fail(to_status(e), why);
}

pkv_status radix_release(pkv_radix* r, int64_t seq) {
  if (!r) return fail(PKV_ERR_ARG, "radix_release: NULL cache");
  if (!r->pool) return fail(PKV_ERR_ARG, "radix_release: the cache's pool was destroyed");
  std::string why;
  pkv::Err e = r->cache.release(seq, &why);
  return e == pkv::Err::ok ? PKV_OK : fail(to_status(e), why);
}

pkv_status radix_evict(pkv_radix* r, int32_t want_free, int32_t* n_free) {
  if (!r) return fail(PKV_ERR_ARG, "radix_evict: NULL cache");
  if (!r->pool) return fail(PKV_ERR_ARG, "radix_evict: the cache's pool was destroyed");
  const bool ok = r->cache.evict(want_free);
  if (n_free) *n_free = static_cast<int32_t>(r->pool->core.free_list().size());
  return ok ? PKV_OK
            : fail(PKV_ERR_OOM, "radix_evict: every remaining cached block is under a live match");
}

pkv_status radix_stats(const pkv_radix* r, int32_t* nodes, int32_t* cached_blocks,
                       int32_t* locked_nodes) {
  if (!r) return fail(PKV_ERR_ARG, "radix_stats: NULL cache");
  if (!r->pool) return fail(PKV_ERR_ARG, "radix_stats: the cache's pool was destroyed");
  if (nodes) *nodes = r->cache.nodes();
  if (cached_blocks) *cached_blocks = r->cache.cached_blocks();
  if (locked_nodes) *locked_nodes = r->cache.locked_nodes();
  return PKV_OK;
}

pkv_status radix_dump(const pkv_radix* r, int32_t* out, int32_t cap, int32_t* n) {
  if (!r || !n) return fail(PKV_ERR_ARG, "radix_dump: NULL argument");
  if (!r->pool) return fail(PKV_ERR_ARG, "radix_dump: the cache's pool was destroyed");
  if (cap > 0 && !out) return fail(PKV_ERR_ARG, "radix_dump: NULL out with cap > 0");
  std::vector<int32_t> d;
  r->cache.dump(&d);
  for (int32_t i = 0; i < static_cast<int32_t>(d.size()) && i < cap; ++i) out[i] = d[i];
  *n = static_cast<int32_t>(d.size());
  return PKV_OK;
}

pkv_status seq_block_table(const pkv_pool* p, int64_t seq, int32_t* out, int32_t cap,
                           int32_t* n_blocks, int32_t* len) {
  if (!p) return fail(PKV_ERR_ARG, "seq_block_table: NULL pool");
  const pkv::SeqState* s = p->core.find(seq);
  if (!s) return fail(PKV_ERR_SEQ, "seq_block_table: unknown sequence " + std::to_string(seq));
  const int32_t n = static_cast<int32_t>(s->table.size());
  if (cap > 0 && !out) return fail(PKV_ERR_ARG, "seq_block_table: NULL out with cap > 0");
  for (int32_t i = 0; i < n && i < cap; ++i) out[i] = s->table[i];
  if (n_blocks) *n_blocks = n;
  if (len) *len = s->len;
  return PKV_OK;
}

pkv_status block_refcount(const pkv_pool* p, int32_t block, int32_t* rc) {
  if (!p || !rc) return fail(PKV_ERR_ARG, "block_refcount: NULL argument");
  if (block < 0 || block >= p->core.shape().num_blocks)
    return fail(PKV_ERR_ARG, "block_refcount: block out of range");
  *rc = p->core.refcount(block);
  return PKV_OK;
}

pkv_status free_list(const pkv_pool* p, int32_t* out, int32_t cap, int32_t* n) {
  if (!p) return fail(PKV_ERR_ARG, "free_list: NULL pool");
  if (cap > 0 && !out) return fail(PKV_ERR_ARG, "free_list: NULL out with cap > 0");
  const auto& f = p->core.free_list();
  int32_t i = 0;
  for (auto it = f.begin(); it != f.end() && i < cap; ++it) out[i++] = *it;
  if (n) *n = static_cast<int32_t>(f.size());
  return PKV_OK;
}

pkv_status kv_last_append(const pkv_pool* p, int32_t* slots, int32_t slot_cap, int32_t* n_slots,
                          int32_t* cow, int32_t cow_cap, int32_t* n_cow) {
  if (!p) return fail(PKV_ERR_ARG, "kv_last_append: NULL pool");
  if ((slot_cap > 0 && !slots) || (cow_cap > 0 && !cow))
    return fail(PKV_ERR_ARG, "kv_last_append: NULL buffer with cap > 0");
  const pkv::AppendResult& r = p->core.last_append();
  const int32_t ns = static_cast<int32_t>(r.slots.size());
  for (int32_t i = 0; i < ns && i < slot_cap; ++i) slots[i] = r.slots[i];
  const int32_t nc = static_cast<int32_t>(r.cow.size());
  for (int32_t i = 0; i < nc && 3 * i + 2 < cow_cap; ++i) {
    cow[3 * i + 0] = r.cow[i].src;
    cow[3 * i + 1] = r.cow[i].dst;
    cow[3 * i + 2] = r.cow[i].n_slots;
  }
  if (n_slots) *n_slots = ns;
  if (n_cow) *n_cow = nc;
  return PKV_OK;
}

}  // extern "C"

namespace {
void fill_stats(const pkv::Plan& plan, const pkv::Shape& sh, pkv_plan_stats* out) {
  out->unique_tokens = plan.unique_tokens;
  out->logical_tokens = plan.logical_tokens;
  out->unique_blocks = plan.unique_blocks;
  out->segments = plan.segments;
  out->work_items = static_cast<int32_t>(plan.valu.size() + plan.mfma.size() + plan.direct.size() +
                                         plan.paths.size());
  out->merged_rows = static_cast<int32_t>(plan.merges.size()) * sh.num_q_heads;
  out->direct = plan.direct.empty() ? 0 : 1;
  out->max_parts = 0;
  for (const pkv::MergeRow& m : plan.merges) out->max_parts = std::max(out->max_parts, m.n_parts);
  out->plan_bytes = static_cast<int64_t>(layout_of(plan).total);
  out->partial_bytes = static_cast<int64_t>(partial_bytes(plan, sh));
}
}  // namespace

extern "C" {

pkv_status paged_attn_decode_plan_stats(pkv_pool* p, const int64_t* seqs, int32_t n_seqs,
                                        pkv_plan_stats* out) {
  if (!p || !out || (n_seqs > 0 && !seqs) || n_seqs < 0)
    return fail(PKV_ERR_ARG, "paged_attn_decode_plan_stats: bad argument");
  pkv::Plan plan;
  std::string why;
  pkv::Err e = pkv::plan_decode(p->core, seqs, n_seqs, p->cfg, &plan, &why);
  if (e != pkv::Err::ok) return fail(to_status(e), why);
  fill_stats(plan, p->core.shape(), out);
  return PKV_OK;
}

pkv_status paged_attn_verify_plan_stats(pkv_pool* p, const int64_t* seqs, int32_t n_seqs, int32_t n_nodes,
                                        const int32_t* parent, pkv_plan_stats* out) {
  if (!p || !out || n_seqs < 1 || !seqs || !parent)
    return fail(PKV_ERR_ARG, "paged_attn_verify_plan_stats: bad argument");
  pkv::Plan plan;
  std::string why;
  pkv::Err e = pkv::plan_verify(p->core, seqs, n_seqs, n_nodes, parent, p->cfg, &plan, &why);
  if (e != pkv::Err::ok) return fail(to_status(e), why);
  fill_stats(plan, p->core.shape(), out);
  return PKV_OK;
}

pkv_status paged_attn_prefill_plan_stats(pkv_pool* p, const int64_t* seqs, int32_t n_seqs, const int32_t* n_new,
                                         pkv_plan_stats* out) {
  if (!p || !out || n_seqs < 1 || !seqs || !n_new)
    return fail(PKV_ERR_ARG, "paged_attn_prefill_plan_stats: bad argument");
  pkv::Plan plan;
  std::string why;
  pkv::Err e = pkv::plan_prefill(p->core, seqs, n_seqs, n_new, p->cfg, &plan, &why);
  if (e != pkv::Err::ok) return fail(to_status(e), why);
  fill_stats(plan, p->core.shape(), out);
  return PKV_OK;
}

pkv_status pkv_hbm_read_probe(const void* src, size_t bytes, void* sink, int32_t blocks, void* stream) {
  if (!src || !sink || blocks < 1 || !aligned16(src) || (bytes & 15))
    return fail(PKV_ERR_ARG, "pkv_hbm_read_probe: NULL buffer, unaligned range or no workgroups");
  PKV_HIP(pkv::launch_read_probe(src, bytes, static_cast<uint32_t*>(sink), blocks,
                                 static_cast<hipStream_t>(stream)));
  return PKV_OK;
}

pkv_status pkv_timing_enable(pkv_pool* p, int32_t enable) {
  if (!p) return fail(PKV_ERR_ARG, "pkv_timing_enable: NULL pool");
  if (!p->device) return fail(PKV_ERR_ARG, "pkv_timing_enable: the pool has no device storage");
  if (enable < 0) return fail(PKV_ERR_ARG, "pkv_timing_enable: negative sampling period");
  p->timing = enable != 0;
  p->timing_every = enable > 0 ? enable : 1;
  p->timing_tick = 0;
  if (!p->timing) {
    for (auto& pr : p->ev_pending) {
      p->ev_free.push_back(pr.first);
      p->ev_free.push_back(pr.second);
    }
    p->ev_pending.clear();
  }
  return PKV_OK;
}

pkv_status pkv_timing_read(pkv_pool* p, double* total_ms, int64_t* calls, int32_t reset) {
  if (!p || !total_ms || !calls) return fail(PKV_ERR_ARG, "pkv_timing_read: NULL argument");
  if (!p->device) return fail(PKV_ERR_ARG, "pkv_timing_read: the pool has no device storage");
  DeviceGuard g(p->dev);
  PKV_HIP(g.err);
  for (auto& pr : p->ev_pending) {
    PKV_HIP(hipEventSynchronize(pr.second));
    float ms = 0.f;
    PKV_HIP(hipEventElapsedTime(&ms, pr.first, pr.second));
    p->timed_ms += ms;
    ++p->timed_calls;
    p->ev_free.push_back(pr.first);
    p->ev_free.push_back(pr.second);
  }
  p->ev_pending.clear();
  *total_ms = p->timed_ms;
  *calls = p->timed_calls;
  if (reset) {
    p->timed_ms = 0.0;
    p->timed_calls = 0;
  }
  return PKV_OK;
}

const char* pkv_last_error(void) { return g_err.c_str(); }

}  // extern "C"
