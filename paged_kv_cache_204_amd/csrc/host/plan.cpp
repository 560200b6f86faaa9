#include "plan.hpp"

#include <algorithm>
#include <climits>
#include <unordered_map>

namespace pkv {
namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Segment {
  std::vector<int32_t> queries;  // indices into the call's query list
  const int32_t* blocks;         // the segment's first block in a member's table
  int32_t nblk;
  int32_t ntok;
  bool ends;                     // the segment holds its queries' last blocks
};

// Chunk length in tokens: spread `work_tokens` (token x row-subset units,
// per kv head) over about `target` workgroups, in multiples of `unit`, within
// [unit, cap].
int32_t pick_chunk(int64_t work_tokens, int32_t kv_heads, int32_t unit, int32_t target,
                   int64_t cap) {
  int64_t per_wg = ceil_div(work_tokens * kv_heads, std::max(1, target));
  int64_t chunk = ceil_div(std::max<int64_t>(per_wg, 1), unit) * unit;
  cap = std::max<int64_t>(unit, (cap / unit) * unit);
  return static_cast<int32_t>(std::min(chunk, cap));
}

int64_t chunk_cap(const PlanConfig& cfg, int32_t block_size) {
  return std::min<int64_t>(cfg.max_chunk, static_cast<int64_t>(cfg.max_chunk_blocks) * block_size);
}

// Lengthens the chunks (by whole multiples of the picked length, in units,
// within the caps) until parts_of(chunk_m, chunk_v), the most partial states
// any query gets, is at most cfg.max_parts or both chunks are at their caps:
// chunks picked for parallelism alone can cut a long shared prefix into so
// many pieces that merging them costs more than the attention itself.
template <class PartsOf>
void limit_parts(const PlanConfig& cfg, int32_t unit, int64_t cap_m, int64_t cap_v, int32_t* chunk_m,
                 int32_t* chunk_v, PartsOf parts_of) {
  if (cfg.max_parts <= 0) return;
  const int32_t m0 = *chunk_m, v0 = *chunk_v;
  for (int32_t f = 2; parts_of(*chunk_m, *chunk_v) > cfg.max_parts; ++f) {
    if (*chunk_m >= cap_m && *chunk_v >= cap_v) break;
    auto grow = [&](int32_t c0, int64_t cap) {
      const int64_t c = ceil_div(static_cast<int64_t>(c0) * f, unit) * unit;
      return static_cast<int32_t>(std::min(c, std::max<int64_t>(unit, (cap / unit) * unit)));
    };
    *chunk_m = grow(m0, cap_m);
    *chunk_v = grow(v0, cap_v);
  }
}

// Waves per MFMA workgroup: eight (one K/V tile staged for 256 rows) only
// when the launch has no VALU items and some query tile fills 256 rows.
int32_t pick_waves(const PlanConfig& cfg, bool any_valu, int32_t row_tiles, int64_t max_rows) {
  if (cfg.mfma_waves == 4 || cfg.mfma_waves == 8) return any_valu || row_tiles != 2 ? 4 : cfg.mfma_waves;
  return !any_valu && row_tiles == 2 && max_rows >= mfma_item_rows(2, 8) ? 8 : 4;
}

// Partial-row bookkeeping shared by both planners: `owner[g]` is the query
// vector of row group g; items that do not cover all keys of their queries
// get partial rows, and every such query gets a merge row.
void finish_parts(Plan* plan, const std::vector<int32_t>& n_parts, int32_t hq) {
  // longest items first within each kind: the kernel starts them first
  auto longer = [](const WorkItem& a, const WorkItem& b) { return a.n_tok > b.n_tok; };
  std::stable_sort(plan->mfma.begin(), plan->mfma.end(), longer);
  std::stable_sort(plan->valu.begin(), plan->valu.end(), longer);
  const size_t nq = n_parts.size();
  // partial rows of every query as one flat list (count, prefix sums, fill):
  // no allocation per query
  auto direct = [&](const WorkItem& it) {
    for (int32_t u = 0; u < it.n_grp; ++u)
      if (n_parts[plan->groups[it.grp_off + u].q_index] != 1) return false;
    return true;
  };
  std::vector<int32_t> start(nq + 1, 0);
  for (const auto* items : {&plan->valu, &plan->mfma})
    for (const WorkItem& it : *items)
      if (!direct(it))
        for (int32_t u = 0; u < it.n_grp; ++u) ++start[plan->groups[it.grp_off + u].q_index + 1];
  for (size_t q = 0; q < nq; ++q) start[q + 1] += start[q];
  std::vector<int32_t> flat(start[nq]);
  std::vector<int32_t> fill(start.begin(), start.end() - 1);
  for (auto* items : {&plan->valu, &plan->mfma}) {
    for (WorkItem& it : *items) {
      if (direct(it)) {
        it.part_base = -1;
        continue;
      }
      it.part_base = static_cast<int32_t>(plan->partial_rows);
      plan->partial_rows += static_cast<int64_t>(it.n_grp) * hq;
      for (int32_t u = 0; u < it.n_grp; ++u)
        flat[fill[plan->groups[it.grp_off + u].q_index]++] = it.part_base + u * hq;
    }
  }
  for (const WorkItem& it : plan->valu) plan->valu_max_rows = std::max(plan->valu_max_rows, it.n_grp);
  std::vector<int32_t> merge_of(nq, -1);
  for (size_t q = 0; q < nq; ++q) {
    if (n_parts[q] <= 1) continue;
    merge_of[q] = static_cast<int32_t>(plan->merges.size());
    MergeRow m{};
    m.q_index = static_cast<int32_t>(q);
    m.n_parts = start[q + 1] - start[q];
    m.parts_off = static_cast<int32_t>(plan->parts.size());
    if (m.n_parts <= kMergeInline)
      std::copy(flat.begin() + start[q], flat.begin() + start[q + 1], m.inl);
    else
      plan->parts.insert(plan->parts.end(), flat.begin() + start[q], flat.begin() + start[q + 1]);
    plan->merges.push_back(m);
  }
  for (RowGroup& g : plan->groups) g.merge = merge_of[g.q_index];
}

// Items (launch order: MFMA, VALU, direct) that end at a query's last key.
void list_tails(Plan* plan) {
  plan->tail_items.clear();
  int32_t k = 0;
  for (const auto* items : {&plan->mfma, &plan->valu, &plan->direct})
    for (const WorkItem& it : *items) {
      if (it.tail_q > 0) plan->tail_items.push_back(k);
      ++k;
    }
}

}  // namespace

// Copies every item's block list to a fixed-stride slot (MFMA items first,
// as the kernel numbers them, then VALU, then direct items), padding with the
// item's last block.
void pack_item_blocks(Plan* plan, int32_t block_size) {
  auto nblk = [&](const WorkItem& it) { return (it.n_tok + block_size - 1) / block_size; };
  plan->stride_mfma = plan->stride_valu = plan->stride_direct = 0;
  for (const WorkItem& it : plan->mfma) plan->stride_mfma = std::max(plan->stride_mfma, nblk(it));
  for (const WorkItem& it : plan->valu) plan->stride_valu = std::max(plan->stride_valu, nblk(it));
  for (const WorkItem& it : plan->direct) plan->stride_direct = std::max(plan->stride_direct, nblk(it));
  plan->item_blocks.assign(plan->mfma.size() * plan->stride_mfma + plan->valu.size() * plan->stride_valu +
                               plan->direct.size() * plan->stride_direct, 0);
  int32_t* dst = plan->item_blocks.data();
  auto put = [&](const std::vector<WorkItem>& items, int32_t stride) {
    for (const WorkItem& it : items) {
      const int32_t n = nblk(it);
      for (int32_t b = 0; b < stride; ++b) dst[b] = plan->blocks[it.blk_off + std::min(b, n - 1)];
      dst += stride;
    }
  };
  put(plan->mfma, plan->stride_mfma);
  put(plan->valu, plan->stride_valu);
  put(plan->direct, plan->stride_direct);
}

bool ancestor_masks(const int32_t* parent, int32_t n_nodes, uint64_t* anc) {
  if (n_nodes < 1 || n_nodes > 64 || !parent || parent[0] != -1) return false;
  anc[0] = 1;
  for (int32_t i = 1; i < n_nodes; ++i) {
    if (parent[i] < 0 || parent[i] >= i) return false;
    anc[i] = anc[parent[i]] | (uint64_t{1} << i);
  }
  return true;
}

Err plan_decode(const BlockPool& pool, const int64_t* seqs, int32_t n_seqs,
                const PlanConfig& cfg, Plan* plan, std::string* why) {
  plan->reset();
  const Shape& sh = pool.shape();
  const int32_t B = sh.block_size;
  const int32_t G = sh.num_q_heads / sh.num_kv_heads;
  std::vector<const SeqState*> st(n_seqs);
  for (int32_t i = 0; i < n_seqs; ++i) {
    st[i] = pool.find(seqs[i]);
    if (!st[i]) {
      *why = "paged_attn_decode: unknown sequence " + std::to_string(seqs[i]);
      return Err::seq;
    }
    if (st[i]->len == 0) {
      *why = "paged_attn_decode: sequence " + std::to_string(seqs[i]) + " is empty";
      return Err::empty;
    }
    plan->logical_tokens += st[i]->len;
    plan->q_epoch.push_back(st[i]->epoch);
    plan->q_len.push_back(st[i]->len);
  }
  auto nblk = [&](int32_t q) { return static_cast<int32_t>(st[q]->table.size()); };
  auto fill = [&](int32_t q, int32_t pos) {
    return std::min(B, st[q]->len - pos * B);
  };

  // ---- trie over block ids, compressed into segments ----
  // A trie node owns the block run [own, e) that its queries share.  A
  // small node (few queries, few tokens, every query continuing below it,
  // not dense enough for the MFMA path) is not made a segment of its own:
  // its run is handed down, so each child's segment starts at the node's
  // start (pos < own) and the run is read once per child instead of costing
  // every query an extra partial state and merge part.
  std::vector<Segment> segs;
  struct Frame {
    std::vector<int32_t> qs;
    int32_t pos;   // first block of the segment this frame emits
    int32_t own;   // first block of the run this frame's queries share
  };
  auto dense = [&](size_t nq) {
    return G > cfg.valu_rows ||
           (cfg.mfma_min_rows > 0 && static_cast<int64_t>(nq) * G >= cfg.mfma_min_rows);
  };
  std::vector<Frame> stack;
  if (cfg.private_segments) {
    // every query its own segment over its whole table: no shared reads,
    // and with the longest chunks the fewest items and partial states
    for (int32_t q = 0; q < n_seqs; ++q) {
      Segment sg;
      sg.queries = {q};
      sg.blocks = st[q]->table.data();
      sg.nblk = nblk(q);
      sg.ntok = st[q]->len;
      sg.ends = true;
      plan->unique_blocks += sg.nblk;
      plan->unique_tokens += sg.ntok;
      segs.push_back(std::move(sg));
    }
  } else if (n_seqs > 0) {
    Frame root;
    root.pos = root.own = 0;
    for (int32_t i = 0; i < n_seqs; ++i) root.qs.push_back(i);
    stack.push_back(std::move(root));
  }
  while (!stack.empty()) {
    Frame f = std::move(stack.back());
    stack.pop_back();
    const std::vector<int32_t>& t0 = st[f.qs[0]]->table;
    int32_t e = f.own;
    for (;;) {
      bool same = true;
      for (int32_t q : f.qs)
        if (nblk(q) <= e || st[q]->table[e] != t0[e]) {
          same = false;
          break;
        }
      if (!same) break;
      ++e;
    }
    bool hand_down = false;
    if (e > f.own) {
      for (int32_t q : f.qs)
        if (fill(q, e - 1) != fill(f.qs[0], e - 1)) {
          *why = "paged_attn_decode: a shared block has different fills (pool invariant broken)";
          return Err::arg;
        }
      plan->unique_blocks += e - f.own;
      plan->unique_tokens += static_cast<int64_t>(e - f.own - 1) * B + fill(f.qs[0], e - 1);
      bool all_continue = true;
      for (int32_t q : f.qs) all_continue = all_continue && nblk(q) > e;
      hand_down = all_continue && !dense(f.qs.size()) &&
                  static_cast<int32_t>(f.qs.size()) <= cfg.unshare_max_queries &&
                  static_cast<int64_t>(e - f.pos) * B <= cfg.unshare_max_tokens;
      if (!hand_down) {
        Segment sg;
        sg.queries = f.qs;
        sg.blocks = t0.data() + f.pos;
        sg.nblk = e - f.pos;
        sg.ntok = (sg.nblk - 1) * B + fill(f.qs[0], e - 1);
        sg.ends = true;
        for (int32_t q : f.qs) sg.ends = sg.ends && nblk(q) == e;
        segs.push_back(std::move(sg));
      }
    }
    // children keyed by the next block id, in first-appearance order
    std::vector<Frame> kids;
    std::unordered_map<int32_t, size_t> index;
    for (int32_t q : f.qs) {
      if (nblk(q) <= e) continue;
      int32_t b = st[q]->table[e];
      auto it = index.find(b);
      if (it == index.end()) {
        index.emplace(b, kids.size());
        kids.push_back(Frame{{q}, hand_down || e == f.own ? f.pos : e, e});
      } else {
        kids[it->second].qs.push_back(q);
      }
    }
    for (auto it = kids.rbegin(); it != kids.rend(); ++it) stack.push_back(std::move(*it));
  }
  plan->segments = static_cast<int32_t>(segs.size());

  // ---- direct plan ----
  // Few, short queries: one item per query over all of its keys.  The
  // kernel then reads a shared prefix once per query (from L2 after the
  // first), but the call is one launch with no partial states; for such
  // calls launch and latency, not bytes, set the time.
  int32_t max_len = 0, max_blocks = 0;
  for (int32_t q = 0; q < n_seqs; ++q) {
    max_len = std::max(max_len, st[q]->len);
    max_blocks = std::max(max_blocks, nblk(q));
  }
  if (cfg.direct_max_tokens > 0 && G <= 16 && max_len <= cfg.direct_max_tokens &&
      max_blocks <= cfg.max_chunk_blocks &&
      static_cast<int64_t>(n_seqs) * sh.num_kv_heads <= cfg.direct_max_wgs) {
    for (int32_t q = 0; q < n_seqs; ++q) {
      WorkItem it{};
      it.blk_off = static_cast<int32_t>(plan->blocks.size());
      it.n_tok = st[q]->len;
      it.tail_start = INT_MAX;
      it.tail_node0 = 0;
      it.grp_off = static_cast<int32_t>(plan->groups.size());
      it.n_grp = 1;
      it.part_base = -1;
      it.tail_q = 1 + q;
      it.q_index[0] = q;
      plan->groups.push_back(RowGroup{q, -1, 0u, 0u, -1, {0, 0, 0}});
      plan->blocks.insert(plan->blocks.end(), st[q]->table.begin(), st[q]->table.end());
      plan->direct.push_back(it);
    }
    std::stable_sort(plan->direct.begin(), plan->direct.end(),
                     [](const WorkItem& a, const WorkItem& b) { return a.n_tok > b.n_tok; });
    pack_item_blocks(plan, B);
    list_tails(plan);
    return Err::ok;
  }

  // ---- tree plan: shared segments through MFMA items, the rest by path items ----
  if (plan_tree(pool, seqs, n_seqs, cfg, plan)) return Err::ok;

  // ---- work items ----
  // Segments read by many rows (a shared prefix under many queries) are a
  // dense contraction and go to the MFMA kernel in row subsets of
  // mfma_item_rows; the rest go to the VALU kernel in subsets of valu_rows.
  // Each kind gets its own key-chunk length.
  auto is_mfma = [&](const Segment& s) {
    return G > cfg.valu_rows ||
           (cfg.mfma_min_rows > 0 && static_cast<int64_t>(s.queries.size()) * G >= cfg.mfma_min_rows);
  };
  bool any_valu = false;
  int64_t max_rows = 0;
  for (const Segment& s : segs) {
    any_valu = any_valu || !is_mfma(s);
    max_rows = std::max<int64_t>(max_rows, static_cast<int64_t>(s.queries.size()) * G);
  }
  plan->mfma_row_tiles = cfg.mfma_row_tiles > 0 ? cfg.mfma_row_tiles : (any_valu ? 1 : 2);
  plan->mfma_waves = pick_waves(cfg, any_valu, plan->mfma_row_tiles, max_rows);
  const int32_t mrows = mfma_item_rows(plan->mfma_row_tiles, plan->mfma_waves);
  const int32_t unit = std::max(cfg.tile, B);
  const int64_t cap = chunk_cap(cfg, B);
  const int64_t cap_v = std::min<int64_t>(cap, cfg.valu_max_tokens);
  int64_t work_v = 0, work_m = 0;
  for (const Segment& s : segs) {
    const bool m = is_mfma(s);
    const int64_t per = std::max(1, (m ? mrows : cfg.valu_rows) / G);
    (m ? work_m : work_v) += static_cast<int64_t>(s.ntok) * ceil_div(static_cast<int64_t>(s.queries.size()), per);
  }
  int32_t chunk_v = pick_chunk(work_v, sh.num_kv_heads, unit, cfg.target_wgs, cap_v);
  int32_t chunk_m = pick_chunk(work_m, sh.num_kv_heads, unit,
                               cfg.target_mfma_wgs * 4 / plan->mfma_waves, cap);
  {
    std::vector<int32_t> parts(n_seqs);
    PlanConfig lim = cfg;
    if (cfg.max_parts > 0 && cfg.wide_max_parts > 0 &&
        static_cast<int64_t>(n_seqs) * sh.num_kv_heads >= cfg.wide_pairs)
      lim.max_parts = std::min(cfg.max_parts, cfg.wide_max_parts);
    limit_parts(lim, unit, cap, cap_v, &chunk_m, &chunk_v, [&](int32_t cm, int32_t cv) {
      std::fill(parts.begin(), parts.end(), 0);
      int32_t most = 0;
      for (const Segment& sg : segs) {
        const int32_t n = static_cast<int32_t>(ceil_div(sg.ntok, is_mfma(sg) ? cm : cv));
        for (int32_t q : sg.queries) most = std::max(most, parts[q] += n);
      }
      return most;
    });
  }

  std::vector<int32_t> n_parts(n_seqs, 0);
  for (const Segment& s : segs) {
    const bool mfma = is_mfma(s);
    const int32_t chunk = mfma ? chunk_m : chunk_v;
    const int32_t per = std::max(1, (mfma ? mrows : cfg.valu_rows) / G);
    const int32_t nchunk = static_cast<int32_t>(ceil_div(s.ntok, chunk));
    for (int32_t q : s.queries) n_parts[q] += nchunk;
    const int32_t blk_base = static_cast<int32_t>(plan->blocks.size());
    plan->blocks.insert(plan->blocks.end(), s.blocks, s.blocks + s.nblk);
    for (size_t u0 = 0; u0 < s.queries.size(); u0 += per) {
      const int32_t ng = static_cast<int32_t>(std::min<size_t>(per, s.queries.size() - u0));
      const int32_t grp_off = static_cast<int32_t>(plan->groups.size());
      for (int32_t u = 0; u < ng; ++u)
        plan->groups.push_back(RowGroup{s.queries[u0 + u], -1, 0u, 0u, -1, {0, 0, 0}});
      for (int32_t c = 0; c < nchunk; ++c) {
        WorkItem it{};
        it.blk_off = blk_base + c * (chunk / B);
        it.n_tok = std::min(chunk, s.ntok - c * chunk);
        it.tail_start = INT_MAX;
        it.tail_node0 = 0;
        it.grp_off = grp_off;
        it.n_grp = ng;
        it.part_base = -1;
        it.tail_q = s.ends && c == nchunk - 1 ? 1 + s.queries[u0] : 0;
        for (int32_t u = 0; u < 8; ++u)
          it.q_index[u] = u < ng ? plan->groups[grp_off + u].q_index : 0;
        (mfma ? plan->mfma : plan->valu).push_back(it);
      }
    }
  }
  finish_parts(plan, n_parts, sh.num_q_heads);
  pack_item_blocks(plan, B);
  list_tails(plan);
  return Err::ok;
}

bool patch_decode(const BlockPool& pool, const int64_t* seqs, int32_t n_seqs, const PlanConfig& cfg,
                  Plan* plan) {
  if (plan->tree || plan->q_epoch.size() != static_cast<size_t>(n_seqs)) return false;
  std::vector<int32_t> grow(n_seqs);
  std::vector<int32_t> last_block(n_seqs);
  for (int32_t q = 0; q < n_seqs; ++q) {
    const SeqState* st = pool.find(seqs[q]);
    if (!st || st->epoch != plan->q_epoch[q] || st->len < plan->q_len[q]) return false;
    if (!plan->direct.empty() && st->len > cfg.direct_max_tokens) return false;
    grow[q] = st->len - plan->q_len[q];
    last_block[q] = st->table.back();
  }
  auto item_at = [&](int32_t k) -> WorkItem& {
    if (k < static_cast<int32_t>(plan->mfma.size())) return plan->mfma[k];
    k -= static_cast<int32_t>(plan->mfma.size());
    if (k < static_cast<int32_t>(plan->valu.size())) return plan->valu[k];
    return plan->direct[k - plan->valu.size()];
  };
  // every query of a tail item ends in the same (unchanged) last block, so
  // all of them grew alike; check it before changing anything
  for (int32_t k : plan->tail_items) {
    const WorkItem& it = item_at(k);
    const int32_t d = grow[it.tail_q - 1];
    for (int32_t u = 0; u < it.n_grp; ++u)
      if (grow[plan->groups[it.grp_off + u].q_index] != d) return false;
  }
  for (int32_t k : plan->tail_items) {
    WorkItem& it = item_at(k);
    it.n_tok += grow[it.tail_q - 1];
  }
  // what the call reads: the new keys of each distinct last block once
  std::vector<std::pair<int32_t, int32_t>> fresh;
  for (int32_t q = 0; q < n_seqs; ++q) {
    plan->logical_tokens += grow[q];
    if (grow[q] > 0) fresh.emplace_back(last_block[q], grow[q]);
    plan->q_len[q] += grow[q];
  }
  std::sort(fresh.begin(), fresh.end());
  fresh.erase(std::unique(fresh.begin(), fresh.end()), fresh.end());
  for (const auto& f : fresh) plan->unique_tokens += f.second;
  return true;
}

Err plan_verify(const BlockPool& pool, const int64_t* seqs, int32_t n_seqs,
                int32_t n_nodes, const int32_t* parent, const PlanConfig& cfg,
                Plan* plan, std::string* why) {
  plan->reset();
  const Shape& sh = pool.shape();
  const int32_t B = sh.block_size;
  const int32_t G = sh.num_q_heads / sh.num_kv_heads;
  if (n_nodes < 1 || n_nodes > 64) {
    *why = "paged_attn_tree_verify: n_nodes must be in 1..64";
    return Err::arg;
  }
  std::vector<const SeqState*> st(n_seqs);
  std::vector<uint64_t> anc(static_cast<size_t>(n_seqs) * n_nodes);
  for (int32_t i = 0; i < n_seqs; ++i) {
    st[i] = pool.find(seqs[i]);
    if (!st[i]) {
      *why = "paged_attn_tree_verify: unknown sequence " + std::to_string(seqs[i]);
      return Err::seq;
    }
    if (st[i]->len < n_nodes) {
      *why = "paged_attn_tree_verify: sequence " + std::to_string(seqs[i]) +
             " is shorter than its tree";
      return Err::arg;
    }
    if (!ancestor_masks(parent + static_cast<size_t>(i) * n_nodes, n_nodes,
                        anc.data() + static_cast<size_t>(i) * n_nodes)) {
      *why = "paged_attn_tree_verify: parent[] of sequence " + std::to_string(i) +
             " is not a tree in node order (parent[0] = -1, 0 <= parent[i] < i)";
      return Err::arg;
    }
  }
  const bool mfma = G > cfg.valu_rows ||
                    (cfg.mfma_min_rows > 0 && static_cast<int64_t>(n_nodes) * G >= cfg.mfma_min_rows);
  plan->mfma_row_tiles = cfg.mfma_row_tiles > 0 ? cfg.mfma_row_tiles : 2;
  plan->mfma_waves = mfma ? pick_waves(cfg, false, plan->mfma_row_tiles,
                                       static_cast<int64_t>(n_nodes) * G)
                          : 4;
  const int32_t per = std::max(1, (mfma ? mfma_item_rows(plan->mfma_row_tiles, plan->mfma_waves)
                                        : cfg.valu_rows) / G);
  const int64_t subsets = ceil_div(n_nodes, per);
  int64_t work = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    work += static_cast<int64_t>(st[i]->len) * subsets;
    plan->unique_tokens += st[i]->len;
    plan->unique_blocks += static_cast<int32_t>(st[i]->table.size());
  }
  plan->segments = n_seqs;
  const int64_t cap = mfma ? chunk_cap(cfg, B)
                           : std::min<int64_t>(chunk_cap(cfg, B), cfg.valu_max_tokens);
  int32_t chunk = pick_chunk(work, sh.num_kv_heads, std::max(cfg.tile, B),
                             mfma ? cfg.target_mfma_wgs * 4 / plan->mfma_waves : cfg.target_wgs,
                             cap);
  {
    int32_t max_len = 0;
    for (int32_t i = 0; i < n_seqs; ++i) max_len = std::max(max_len, st[i]->len);
    int32_t unused = chunk;
    limit_parts(cfg, std::max(cfg.tile, B), cap, cap, &chunk, &unused,
                [&](int32_t c, int32_t) { return static_cast<int32_t>(ceil_div(max_len, c)); });
  }
  std::vector<int32_t> n_parts(static_cast<size_t>(n_seqs) * n_nodes, 0);
  for (int32_t i = 0; i < n_seqs; ++i) {
    const int32_t len = st[i]->len;
    const int32_t ctx = len - n_nodes;
    const int32_t nchunk = static_cast<int32_t>(ceil_div(len, chunk));
    const int32_t blk_base = static_cast<int32_t>(plan->blocks.size());
    plan->blocks.insert(plan->blocks.end(), st[i]->table.begin(), st[i]->table.end());
    for (int32_t j = 0; j < n_nodes; ++j) {
      n_parts[static_cast<size_t>(i) * n_nodes + j] = nchunk;
      // logical keys of node j: the context plus its ancestors and itself
      plan->logical_tokens += ctx + __builtin_popcountll(anc[static_cast<size_t>(i) * n_nodes + j]);
    }
    for (int32_t j0 = 0; j0 < n_nodes; j0 += per) {
      const int32_t ng = std::min(per, n_nodes - j0);
      const int32_t grp_off = static_cast<int32_t>(plan->groups.size());
      for (int32_t j = j0; j < j0 + ng; ++j) {
        uint64_t m = anc[static_cast<size_t>(i) * n_nodes + j];
        plan->groups.push_back(RowGroup{i * n_nodes + j, j, static_cast<uint32_t>(m),
                                        static_cast<uint32_t>(m >> 32), -1, {0, 0, 0}});
      }
      for (int32_t c = 0; c < nchunk; ++c) {
        const int32_t start = c * chunk;
        WorkItem it{};
        it.blk_off = blk_base + start / B;
        it.n_tok = std::min(chunk, len - start);
        if (ctx - start >= it.n_tok) {
          it.tail_start = INT_MAX;
          it.tail_node0 = 0;
        } else if (start >= ctx) {
          it.tail_start = 0;
          it.tail_node0 = start - ctx;
        } else {
          it.tail_start = ctx - start;
          it.tail_node0 = 0;
        }
        it.grp_off = grp_off;
        it.n_grp = ng;
        it.part_base = -1;
        it.tail_q = 0;
        for (int32_t u = 0; u < 8; ++u)
          it.q_index[u] = u < ng ? plan->groups[grp_off + u].q_index : 0;
        (mfma ? plan->mfma : plan->valu).push_back(it);
      }
    }
  }
  finish_parts(plan, n_parts, sh.num_q_heads);
  pack_item_blocks(plan, B);
  return Err::ok;
}

}  // namespace pkv

namespace pkv {

// Causal prefill as chain-shaped key tails: the new tokens of a sequence are
// cut into windows of `per` consecutive queries (at most 64, one item's row
// subset).  A window's key range runs from token 0 to its last query's own
// token; its own tokens are the item's masked tail, node k of the window
// seeing nodes 0..k (the ancestor-or-self mask of a chain), everything before
// the window is unmasked context.  So the kernels' tree-tail masking serves
// the causal mask unchanged, and no window reads keys past its last query.
Err plan_prefill(const BlockPool& pool, const int64_t* seqs, int32_t n_seqs, const int32_t* n_new,
                 const PlanConfig& cfg, Plan* plan, std::string* why) {
  plan->reset();
  const Shape& sh = pool.shape();
  const int32_t B = sh.block_size;
  const int32_t G = sh.num_q_heads / sh.num_kv_heads;
  std::vector<const SeqState*> st(n_seqs);
  std::vector<int32_t> q_off(static_cast<size_t>(n_seqs) + 1, 0);
  int32_t max_new = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    st[i] = pool.find(seqs[i]);
    if (!st[i]) {
      *why = "paged_attn_prefill: unknown sequence " + std::to_string(seqs[i]);
      return Err::seq;
    }
    if (n_new[i] < 0 || n_new[i] > st[i]->len) {
      *why = "paged_attn_prefill: sequence " + std::to_string(seqs[i]) + " holds " +
             std::to_string(st[i]->len) + " tokens, fewer than its " + std::to_string(n_new[i]) +
             " new ones (or the count is negative)";
      return Err::arg;
    }
    if (static_cast<int64_t>(q_off[i]) + n_new[i] > kMaxPrefillQueries) {
      *why = "paged_attn_prefill: more than " + std::to_string(kMaxPrefillQueries) + " queries in one call";
      return Err::arg;
    }
    q_off[i + 1] = q_off[i] + n_new[i];
    max_new = std::max(max_new, n_new[i]);
  }
  const int32_t nq = q_off[n_seqs];
  if (nq == 0) return Err::ok;
  const int64_t win_rows = static_cast<int64_t>(std::min(max_new, 64)) * G;
  const bool mfma = G > cfg.valu_rows || (cfg.mfma_min_rows > 0 && win_rows >= cfg.mfma_min_rows);
  plan->mfma_row_tiles = cfg.mfma_row_tiles > 0 ? cfg.mfma_row_tiles : 2;
  plan->mfma_waves = mfma ? pick_waves(cfg, false, plan->mfma_row_tiles, win_rows) : 4;
  const int32_t per = std::min(
      64, std::max(1, (mfma ? mfma_item_rows(plan->mfma_row_tiles, plan->mfma_waves) : cfg.valu_rows) / G));
  // work (tokens x windows, per kv head) and what the call reads: the
  // distinct blocks of the sequences with new tokens, at their filled slots
  int64_t work = 0;
  int32_t max_len = 0;
  std::vector<int32_t> filled(static_cast<size_t>(sh.num_blocks), 0);
  for (int32_t i = 0; i < n_seqs; ++i) {
    const int32_t n = n_new[i];
    if (n == 0) continue;
    const int32_t len = st[i]->len;
    const int32_t ctx = len - n;
    max_len = std::max(max_len, len);
    for (int32_t w0 = 0; w0 < n; w0 += per) work += ctx + std::min(n, w0 + per);
    for (int32_t j = 0; j < n; ++j) plan->logical_tokens += ctx + j + 1;
    const auto& t = st[i]->table;
    for (size_t b = 0; b < t.size(); ++b)
      filled[t[b]] = std::max(filled[t[b]], std::min<int32_t>(B, len - static_cast<int32_t>(b) * B));
  }
  for (int32_t f : filled) {
    plan->unique_tokens += f;
    plan->unique_blocks += f > 0;
  }
  const int64_t cap = mfma ? chunk_cap(cfg, B) : std::min<int64_t>(chunk_cap(cfg, B), cfg.valu_max_tokens);
  const int32_t unit = std::max(cfg.tile, B);
  int32_t chunk = pick_chunk(work, sh.num_kv_heads, unit,
                             mfma ? cfg.target_mfma_wgs * 4 / plan->mfma_waves : cfg.target_wgs, cap);
  {
    int32_t unused = chunk;
    limit_parts(cfg, unit, cap, cap, &chunk, &unused,
                [&](int32_t c, int32_t) { return static_cast<int32_t>(ceil_div(max_len, c)); });
  }
  std::vector<int32_t> n_parts(static_cast<size_t>(nq), 0);
  for (int32_t i = 0; i < n_seqs; ++i) {
    const int32_t n = n_new[i];
    if (n == 0) continue;
    const int32_t len = st[i]->len;
    const int32_t ctx = len - n;
    const int32_t blk_base = static_cast<int32_t>(plan->blocks.size());
    plan->blocks.insert(plan->blocks.end(), st[i]->table.begin(), st[i]->table.end());
    for (int32_t w0 = 0; w0 < n; w0 += per) {
      const int32_t nw = std::min(per, n - w0);
      const int32_t tail = ctx + w0;         // the window's first own token
      const int32_t end = tail + nw;         // keys of the window: 0 .. end - 1
      const int32_t nchunk = static_cast<int32_t>(ceil_div(end, chunk));
      const int32_t grp_off = static_cast<int32_t>(plan->groups.size());
      for (int32_t k = 0; k < nw; ++k) {
        const uint64_t m = k == 63 ? ~0ull : (2ull << k) - 1;   // nodes 0..k of the window
        plan->groups.push_back(RowGroup{q_off[i] + w0 + k, k, static_cast<uint32_t>(m),
                                        static_cast<uint32_t>(m >> 32), -1, {0, 0, 0}});
        n_parts[q_off[i] + w0 + k] = nchunk;
      }
      for (int32_t c = 0; c < nchunk; ++c) {
        const int32_t start = c * chunk;
        WorkItem it{};
        it.blk_off = blk_base + start / B;
        it.n_tok = std::min(chunk, end - start);
        if (tail - start >= it.n_tok) {
          it.tail_start = INT_MAX;
          it.tail_node0 = 0;
        } else if (start >= tail) {
          it.tail_start = 0;
          it.tail_node0 = start - tail;
        } else {
          it.tail_start = tail - start;
          it.tail_node0 = 0;
        }
        it.grp_off = grp_off;
        it.n_grp = nw;
        it.part_base = -1;
        it.tail_q = 0;
        for (int32_t u = 0; u < 8; ++u) it.q_index[u] = u < nw ? plan->groups[grp_off + u].q_index : 0;
        (mfma ? plan->mfma : plan->valu).push_back(it);
      }
    }
  }
  plan->segments = n_seqs;
  finish_parts(plan, n_parts, sh.num_q_heads);
  pack_item_blocks(plan, B);
  return Err::ok;
}

}  // namespace pkv
