// Replays an op list (stdin, the format of plan_patch_check.cpp: "shape ...",
// "alloc h", "fork a b", "append n h...", "free h", "decode h...") through the
// host pool and plans every decode call.  Each tree plan is checked against
// the tables themselves:
//  - every query is in exactly one path item, at most 32 rows each;
//  - the keys of a query -- tokens of the MFMA items that list it, plus the
//    tokens of the steps of its path item whose mask names it -- are exactly
//    the (block, slot) pairs of its table for tokens 0 .. len-1, each once;
//  - its merge row lists exactly the partial rows of those MFMA items;
//  - steps stay inside their blocks.
// Prints "tree T other O" and exits 1 on the first mismatch.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <iostream>
#include <map>
#include <sstream>
#include <string>
#include <vector>

#include "host/plan.hpp"

using namespace pkv;

static int fail(const std::string& what) {
  std::printf("FAIL %s\n", what.c_str());
  return 1;
}

static std::string check(const BlockPool& pool, const std::vector<int64_t>& ids, const Plan& plan) {
  const Shape& sh = pool.shape();
  const int32_t B = sh.block_size, G = sh.num_q_heads / sh.num_kv_heads;
  const size_t nq = ids.size();
  std::vector<std::vector<std::pair<int32_t, int32_t>>> got(nq);
  std::vector<std::vector<int32_t>> parts(nq);
  std::vector<int> in_path(nq, 0);
  for (size_t i = 0; i < plan.mfma.size(); ++i) {
    const WorkItem& it = plan.mfma[i];
    const int32_t* lst = plan.item_blocks.data() + i * plan.stride_mfma;
    if (it.part_base < 0) return "an MFMA item writes final output";
    if (it.n_grp * G > 256) return "an MFMA item over 256 rows";
    for (int32_t u = 0; u < it.n_grp; ++u) {
      const int32_t q = plan.groups[it.grp_off + u].q_index;
      parts[q].push_back(it.part_base + u * sh.num_q_heads);
      for (int32_t t = 0; t < it.n_tok; ++t) got[q].emplace_back(lst[t / B], t % B);
    }
  }
  for (const PathItem& pi : plan.paths) {
    if (pi.n_q < 1 || pi.n_q > kPathMaxQ || pi.n_q * G > kPathMaxRows) return "a path item's rows";
    for (int32_t j = 0; j < pi.n_q; ++j) {
      const int32_t q = pi.q_index[j];
      ++in_path[q];
      std::vector<int32_t> want = parts[q];
      std::vector<int32_t> have;
      if (pi.merge[j] >= 0) {
        const MergeRow& m = plan.merges[pi.merge[j]];
        if (m.q_index != q || m.n_parts > kPathMaxParts) return "merge row";
        have.assign(m.inl, m.inl + m.n_parts);
      }
      std::sort(want.begin(), want.end());
      std::sort(have.begin(), have.end());
      if (want != have) return "a query's merge row does not list its partial rows";
    }
    for (int32_t s = pi.step_off; s < pi.step_off + pi.n_steps; ++s) {
      const PathStep& ps = plan.steps[s];
      const int32_t off = ps.meta & 0xFF, n = (ps.meta >> 8) & 0xFF;
      if (n < 1 || n > 32) return "step token count";
      if (B == 16 ? off != 0 : (off + n > B || ps.blk_a != ps.blk_b)) return "step leaves its block";
      if (pi.n_q < 32 && (ps.qmask >> pi.n_q)) return "step mask names a query outside the item";
      for (int32_t j = 0; j < pi.n_q; ++j) {
        if (!((ps.qmask >> j) & 1u)) continue;
        for (int32_t t = 0; t < n; ++t)
          got[pi.q_index[j]].emplace_back(t < 16 ? ps.blk_a : ps.blk_b, (off + t) & (B - 1));
      }
    }
  }
  for (size_t q = 0; q < nq; ++q) {
    if (in_path[q] != 1) return "query " + std::to_string(q) + " is in " + std::to_string(in_path[q]) + " path items";
    const SeqState* st = pool.find(ids[q]);
    std::vector<std::pair<int32_t, int32_t>> want;
    for (int32_t t = 0; t < st->len; ++t) want.emplace_back(st->table[t / B], t % B);
    std::sort(want.begin(), want.end());
    std::sort(got[q].begin(), got[q].end());
    if (want != got[q]) return "query " + std::to_string(q) + ": keys covered differ from its table";
  }
  return "";
}

int main() {
  std::string line, w;
  std::getline(std::cin, line);
  std::istringstream hs(line);
  Shape sh{};
  hs >> w >> sh.num_blocks >> sh.block_size >> sh.num_layers >> sh.num_q_heads >> sh.num_kv_heads >>
      sh.head_dim;
  BlockPool pool(sh, nullptr);
  std::map<int, int64_t> h;
  std::string why;
  PlanConfig cfg;
  cfg.direct_max_tokens = 0;   // every call planned as segments or as a tree
  cfg.tree_min_wgs = 0;        // small batches too
  if (const char* e = std::getenv("TREE_CHECK_WIDE_ROWS")) cfg.tree_wide_rows = std::atoi(e);
  if (const char* e = std::getenv("TREE_CHECK_WIDE_TOKENS")) cfg.tree_wide_tokens = std::atoi(e);
  if (const char* e = std::getenv("TREE_CHECK_PATH_TOKENS")) cfg.tree_path_tokens = std::atoi(e);
  if (const char* e = std::getenv("TREE_CHECK_MAX_PARTS")) cfg.tree_max_parts = std::atoi(e);
  if (const char* e = std::getenv("TREE_CHECK_MIN_WGS")) cfg.tree_min_wgs = std::atoi(e);
  int trees = 0, others = 0;
  while (std::getline(std::cin, line)) {
    std::istringstream ls(line);
    ls >> w;
    if (w == "alloc") {
      int a;
      ls >> a;
      h[a] = pool.allocate();
    } else if (w == "fork") {
      int a, b;
      ls >> a >> b;
      int64_t c;
      if (pool.fork(h[a], &c, &why) != Err::ok) return fail(why);
      h[b] = c;
    } else if (w == "free") {
      int a;
      ls >> a;
      if (pool.release(h[a], &why) != Err::ok) return fail(why);
      h.erase(a);
    } else if (w == "append") {
      int n, a;
      ls >> n;
      std::vector<int64_t> ids;
      while (ls >> a) ids.push_back(h[a]);
      PendingAppend pa;
      if (pool.prepare_append(ids.data(), static_cast<int32_t>(ids.size()), n, &pa, &why) != Err::ok)
        return fail(why);
      pool.commit_append(std::move(pa));
    } else if (w == "decode") {
      int a;
      std::vector<int64_t> ids;
      while (ls >> a) ids.push_back(h[a]);
      Plan plan;
      if (plan_decode(pool, ids.data(), static_cast<int32_t>(ids.size()), cfg, &plan, &why) != Err::ok)
        return fail(why);
      if (!plan.tree) {
        ++others;
        continue;
      }
      ++trees;
      const std::string err = check(pool, ids, plan);
      if (!err.empty()) return fail(err);
    }
  }
  std::printf("tree %d other %d\n", trees, others);
  return 0;
}
