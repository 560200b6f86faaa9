// Replays an op list (stdin: "shape ...", "alloc h", "fork a b", "append n h...",
// "free h", "decode h...") through the host pool.  The first decode of a
// sequence list is planned; each later decode of the same list is patched
// (patch_decode) when its tables are unchanged and replanned otherwise.
// Every plan is checked: the items covering each query tile exactly
// [0, len) of its keys, and a patched plan's read counts equal a fresh
// plan's.  Prints "patched P replanned R" and exits 1 on the first mismatch.
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

// keys each query's items cover (sum of n_tok over the items listing it)
static std::vector<long> coverage(const Plan& plan, size_t n_q) {
  std::vector<long> cov(n_q, 0);
  for (const auto* items : {&plan.mfma, &plan.valu, &plan.direct})
    for (const WorkItem& it : *items)
      for (int32_t u = 0; u < it.n_grp; ++u) cov[plan.groups[it.grp_off + u].q_index] += it.n_tok;
  return cov;
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
  cfg.tree_decode = 0;   // tree plans are replanned, never patched: the segment planner here
  if (const char* e = std::getenv("PATCH_CHECK_DIRECT")) cfg.direct_max_tokens = std::atoi(e);
  Plan cached;
  std::vector<int64_t> cached_ids;
  int patched = 0, replanned = 0;
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
    } else if (w == "append") {
      int n, x;
      ls >> n;
      std::vector<int64_t> ids;
      while (ls >> x) ids.push_back(h[x]);
      PendingAppend pa;
      if (pool.prepare_append(ids.data(), static_cast<int32_t>(ids.size()), n, &pa, &why) != Err::ok)
        return fail(why);
      pool.commit_append(std::move(pa));
    } else if (w == "decode") {
      int x;
      std::vector<int64_t> ids;
      while (ls >> x) ids.push_back(h[x]);
      const int32_t n = static_cast<int32_t>(ids.size());
      Plan fresh;
      if (plan_decode(pool, ids.data(), n, cfg, &fresh, &why) != Err::ok) return fail(why);
      if (ids == cached_ids && patch_decode(pool, ids.data(), n, cfg, &cached)) {
        ++patched;
        if (cached.unique_tokens != fresh.unique_tokens || cached.logical_tokens != fresh.logical_tokens)
          return fail("patched read counts differ from a fresh plan");
      } else {
        ++replanned;
        cached = fresh;
        cached_ids = ids;
      }
      const std::vector<long> cov = coverage(cached, ids.size());
      for (int32_t q = 0; q < n; ++q)
        if (cov[q] != pool.find(ids[q])->len)
          return fail("query " + std::to_string(q) + " covers " + std::to_string(cov[q]) + " keys of " +
                      std::to_string(pool.find(ids[q])->len));
    }
  }
  std::printf("patched %d replanned %d\n", patched, replanned);
  return 0;
}
