// Tree decode plans: a decode call over prefix-sharing sequences (branches
// of a search tree, forks of one prompt) as two kinds of work.
//
// The batch's block tables form a trie keyed by physical block id: a node is
// a maximal run of blocks that one set of queries shares (the radix-tree view
// of shared prefixes, SGLang RadixAttention page, data-structure foundations
// and the match / split operations; keyed on the blocks the pool already
// shares, so no token comparison is needed).
//  - The queries in trie order are cut into groups of whole queries of at
//    most 32 rows (queries x the G query heads of a kv head); a group's path
//    item walks the nodes on its queries' paths, root first, in 32-token
//    steps, each step carrying the mask of the group's queries that see it.
//    Siblings are adjacent in trie order, so the narrow levels of a search
//    tree are read once per group and a leaf's own keys once; a shared run
//    is read by every group below it, at the same time, so for a run of a
//    few thousand keys (a few MB over all kv heads) the repeats come from
//    the L2 cache of the XCD running that kv head, not from HBM.  No partial
//    states and no merge: each path item writes its rows of out / lse.
//  - A run longer than tree_path_tokens, or read by at least tree_wide_rows
//    rows over at least tree_wide_tokens keys, is instead a dense
//    contraction: MFMA items of up to tree_item_rows rows x one key chunk
//    each, writing partial softmax states in a launch before the path items,
//    which merge them into their rows by log-sum-exp.
#include <algorithm>
#include <climits>
#include <unordered_map>

#include "plan.hpp"

namespace pkv {
namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Node {
  int32_t parent;            // -1: a top-level node
  int32_t pos;               // first block position of the run in its members' tables
  int32_t nblk;
  int32_t ntok;              // keys of the run (the last block may be partial)
  const int32_t* blocks;     // the run in one member's table
  std::vector<int32_t> qs;   // queries whose keys include the run
  bool wide = false;
};

}  // namespace

bool plan_tree(const BlockPool& pool, const int64_t* seqs, int32_t n_seqs, const PlanConfig& cfg,
               Plan* out) {
  const Shape& sh = pool.shape();
  const int32_t B = sh.block_size;
  const int32_t G = sh.num_q_heads / sh.num_kv_heads;
  if (cfg.tree_decode <= 0 || B < 16 || G > 16 || n_seqs < 1) return false;
  const int32_t max_parts = std::min(cfg.tree_max_parts, kPathMaxParts);
  if (max_parts < 1) return false;
  std::vector<const SeqState*> st(n_seqs);
  for (int32_t i = 0; i < n_seqs; ++i) {
    st[i] = pool.find(seqs[i]);
    if (!st[i] || st[i]->len == 0) return false;
  }
  auto nblk = [&](int32_t q) { return static_cast<int32_t>(st[q]->table.size()); };
  auto fill = [&](int32_t q, int32_t pos) { return std::min(B, st[q]->len - pos * B); };

  // ---- trie over the block tables, in preorder ----
  std::vector<Node> nodes;
  std::vector<int32_t> q_order;          // queries in trie order (where their tables end)
  std::vector<int32_t> q_end(n_seqs, -1);  // node holding a query's last block
  struct Frame {
    std::vector<int32_t> qs;
    int32_t own;
    int32_t parent;
  };
  std::vector<Frame> stack;
  {
    Frame root;
    root.own = 0;
    root.parent = -1;
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
    int32_t here = f.parent;
    if (e > f.own) {
      for (int32_t q : f.qs)
        if (fill(q, e - 1) != fill(f.qs[0], e - 1)) return false;   // pool invariant broken
      Node nd;
      nd.parent = f.parent;
      nd.pos = f.own;
      nd.nblk = e - f.own;
      nd.ntok = (nd.nblk - 1) * B + fill(f.qs[0], e - 1);
      nd.blocks = t0.data() + f.own;
      nd.qs = f.qs;
      here = static_cast<int32_t>(nodes.size());
      nodes.push_back(std::move(nd));
      for (int32_t q : f.qs)
        if (nblk(q) == e) {
          q_end[q] = here;
          q_order.push_back(q);
        }
    }
    std::vector<Frame> kids;
    std::unordered_map<int32_t, size_t> index;
    for (int32_t q : f.qs) {
      if (nblk(q) <= e) continue;
      const int32_t b = st[q]->table[e];
      auto it = index.find(b);
      if (it == index.end()) {
        index.emplace(b, kids.size());
        kids.push_back(Frame{{q}, e, here});
      } else {
        kids[it->second].qs.push_back(q);
      }
    }
    for (auto it = kids.rbegin(); it != kids.rend(); ++it) stack.push_back(std::move(*it));
  }
  if (static_cast<int32_t>(q_order.size()) != n_seqs) return false;

  // ---- which nodes are shared through MFMA items ----
  bool any_wide = false;
  for (Node& nd : nodes) {
    const int64_t rows = static_cast<int64_t>(nd.qs.size()) * G;
    nd.wide = (rows >= cfg.tree_wide_rows && nd.ntok >= cfg.tree_wide_tokens) ||
              nd.ntok > cfg.tree_path_tokens;
    any_wide = any_wide || nd.wide;
  }
  const int32_t item_rows = std::max(16, std::min(256, cfg.tree_item_rows));
  const int32_t per = std::max(1, item_rows / G);     // queries per MFMA item
  const int32_t unit = std::max(64, B);
  const int64_t cap = std::max<int64_t>(
      unit, std::min<int64_t>(cfg.max_chunk, static_cast<int64_t>(cfg.max_chunk_blocks) * B) / unit * unit);
  int32_t chunk = static_cast<int32_t>(unit);
  std::vector<int32_t> parts(n_seqs, 0);
  if (any_wide) {
    int64_t work = 0;   // tokens x row subsets, per kv head
    for (const Node& nd : nodes)
      if (nd.wide) work += static_cast<int64_t>(nd.ntok) * ceil_div(static_cast<int64_t>(nd.qs.size()), per);
    const int64_t per_wg = ceil_div(work * sh.num_kv_heads, std::max(1, cfg.tree_target_wgs));
    chunk = static_cast<int32_t>(std::min<int64_t>(cap, std::max<int64_t>(unit, ceil_div(per_wg, unit) * unit)));
    // fewer, longer chunks until no query has more than max_parts partial states
    for (;;) {
      std::fill(parts.begin(), parts.end(), 0);
      int32_t most = 0;
      for (const Node& nd : nodes) {
        if (!nd.wide) continue;
        const int32_t n = static_cast<int32_t>(ceil_div(nd.ntok, chunk));
        for (int32_t q : nd.qs) most = std::max(most, parts[q] += n);
      }
      if (most <= max_parts) break;
      if (chunk >= cap) return false;
      chunk = static_cast<int32_t>(std::min<int64_t>(cap, static_cast<int64_t>(chunk) * 2));
    }
  }

  Plan plan;
  plan.tree = true;
  plan.mfma_row_tiles = 2;
  plan.mfma_waves = 8;

  // ---- MFMA items over the wide nodes, partial rows per query ----
  std::vector<std::vector<int32_t>> q_parts(n_seqs);
  for (const Node& nd : nodes) {
    if (!nd.wide) continue;
    const int32_t nchunk = static_cast<int32_t>(ceil_div(nd.ntok, chunk));
    const int32_t blk_base = static_cast<int32_t>(plan.blocks.size());
    plan.blocks.insert(plan.blocks.end(), nd.blocks, nd.blocks + nd.nblk);
    for (size_t u0 = 0; u0 < nd.qs.size(); u0 += per) {
      const int32_t ng = static_cast<int32_t>(std::min<size_t>(per, nd.qs.size() - u0));
      const int32_t grp_off = static_cast<int32_t>(plan.groups.size());
      for (int32_t u = 0; u < ng; ++u) plan.groups.push_back(RowGroup{nd.qs[u0 + u], -1, 0u, 0u, -1, {0, 0, 0}});
      for (int32_t c = 0; c < nchunk; ++c) {
        WorkItem it{};
        it.blk_off = blk_base + c * (chunk / B);
        it.n_tok = std::min(chunk, nd.ntok - c * chunk);
        it.tail_start = INT_MAX;
        it.tail_node0 = 0;
        it.grp_off = grp_off;
        it.n_grp = ng;
        it.part_base = static_cast<int32_t>(plan.partial_rows);
        it.tail_q = 0;
        for (int32_t u = 0; u < 8; ++u) it.q_index[u] = u < ng ? nd.qs[u0 + u] : 0;
        plan.partial_rows += static_cast<int64_t>(ng) * sh.num_q_heads;
        for (int32_t u = 0; u < ng; ++u) q_parts[nd.qs[u0 + u]].push_back(it.part_base + u * sh.num_q_heads);
        plan.mfma.push_back(it);
      }
    }
  }
  // longest items first: the kernel starts them first
  std::stable_sort(plan.mfma.begin(), plan.mfma.end(),
                   [](const WorkItem& a, const WorkItem& b) { return a.n_tok > b.n_tok; });
  std::vector<int32_t> merge_of(n_seqs, -1);
  for (int32_t q = 0; q < n_seqs; ++q) {
    if (q_parts[q].empty()) continue;
    merge_of[q] = static_cast<int32_t>(plan.merges.size());
    MergeRow m{};
    m.q_index = q;
    m.n_parts = static_cast<int32_t>(q_parts[q].size());
    m.parts_off = 0;
    std::copy(q_parts[q].begin(), q_parts[q].end(), m.inl);
    plan.merges.push_back(m);
  }

  // ---- path items: groups of whole queries in trie order ----
  const int32_t qp = std::max(1, std::min(kPathMaxQ, kPathMaxRows / G));
  std::vector<int32_t> mark(nodes.size(), -1);   // node -> index in the item's node list
  std::vector<int32_t> item_nodes;
  std::vector<uint32_t> item_mask;
  for (size_t g0 = 0; g0 < q_order.size(); g0 += qp) {
    const int32_t nq = static_cast<int32_t>(std::min<size_t>(qp, q_order.size() - g0));
    PathItem pi{};
    pi.step_off = static_cast<int32_t>(plan.steps.size());
    pi.n_q = nq;
    for (int32_t j = 0; j < kPathMaxQ; ++j) {
      pi.q_index[j] = j < nq ? q_order[g0 + j] : 0;
      pi.merge[j] = j < nq ? merge_of[q_order[g0 + j]] : -1;
    }
    item_nodes.clear();
    item_mask.clear();
    for (int32_t j = 0; j < nq; ++j)
      for (int32_t nd = q_end[q_order[g0 + j]]; nd >= 0; nd = nodes[nd].parent) {
        if (nodes[nd].wide) continue;
        if (mark[nd] < 0) {
          mark[nd] = static_cast<int32_t>(item_nodes.size());
          item_nodes.push_back(nd);
          item_mask.push_back(0);
        }
        item_mask[mark[nd]] |= 1u << j;
      }
    // root first (node ids are in preorder)
    std::vector<size_t> order(item_nodes.size());
    for (size_t k = 0; k < order.size(); ++k) order[k] = k;
    std::sort(order.begin(), order.end(), [&](size_t a, size_t b) { return item_nodes[a] < item_nodes[b]; });
    for (size_t k : order) {
      const Node& nd = nodes[item_nodes[k]];
      for (int32_t t0 = 0; t0 < nd.ntok; t0 += 32) {
        PathStep ps{};
        const int32_t bi = t0 / B;
        ps.blk_a = nd.blocks[bi];
        ps.blk_b = (B == 16 && t0 + 16 < nd.ntok) ? nd.blocks[bi + 1] : ps.blk_a;
        ps.meta = (t0 % B) | (std::min(32, nd.ntok - t0) << 8);
        ps.qmask = item_mask[k];
        plan.steps.push_back(ps);
      }
    }
    for (int32_t nd : item_nodes) mark[nd] = -1;
    pi.n_steps = static_cast<int32_t>(plan.steps.size()) - pi.step_off;
    plan.paths.push_back(pi);
  }
  // a batch too small to fill the chip this way goes to the segment planner
  if (static_cast<int64_t>(plan.paths.size()) * sh.num_kv_heads < cfg.tree_min_wgs) return false;

  plan.segments = static_cast<int32_t>(nodes.size());
  pack_item_blocks(&plan, B);
  // what the call reads and the sequences it was made for stay the caller's
  plan.unique_tokens = out->unique_tokens;
  plan.logical_tokens = out->logical_tokens;
  plan.unique_blocks = out->unique_blocks;
  plan.q_epoch = std::move(out->q_epoch);
  plan.q_len = std::move(out->q_len);
  *out = std::move(plan);
  return true;
}

}  // namespace pkv
