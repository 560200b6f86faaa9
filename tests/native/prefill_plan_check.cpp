// Random prefill calls through the host planner (no GPU).  For every plan:
// each (query, key) pair the items let through -- a key inside an item's
// range, before its tail or in the row's ancestor-or-self mask -- must be a
// causal pair (key position <= query position), every causal pair must be
// let through exactly once, mask shifts stay below 64, item rows and block
// lists fit the kernels' limits, and the block an item reads for a key is
// the sequence's own block for that position.
// Usage: prefill_plan_check SEED ROUNDS; prints "ok N plans" or "FAIL ...".
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <string>
#include <utility>
#include <vector>

#include "host/plan.hpp"

using namespace pkv;

static int fail(const std::string& what) {
  std::printf("FAIL %s\n", what.c_str());
  return 1;
}

int main(int argc, char** argv) {
  const unsigned seed = argc > 1 ? std::atoi(argv[1]) : 1;
  const int rounds = argc > 2 ? std::atoi(argv[2]) : 50;
  std::mt19937 rng(seed);
  auto pick = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  int plans = 0;
  for (int r = 0; r < rounds; ++r) {
    const int Bs[] = {1, 2, 4, 16, 32, 64};
    const int Gs[] = {1, 2, 4, 8, 16};
    Shape sh{};
    sh.block_size = Bs[pick(0, 5)];
    sh.num_kv_heads = pick(1, 4);
    sh.num_q_heads = sh.num_kv_heads * Gs[pick(0, 4)];
    sh.head_dim = 64;
    sh.num_layers = 1;
    sh.num_blocks = 4096;
    BlockPool pool(sh, nullptr);
    PlanConfig cfg;
    if (pick(0, 3) == 0) cfg.mfma_min_rows = 0;
    if (pick(0, 3) == 0) cfg.target_mfma_wgs = pick(1, 64);
    if (pick(0, 3) == 0) cfg.target_wgs = pick(1, 64);
    std::string why;
    // a shared root, forks that append their own prompts
    const int64_t root = pool.allocate();
    const int root_len = pick(0, 300);
    auto append = [&](int64_t s, int n_tok) {
      PendingAppend pa;
      if (pool.prepare_append(&s, 1, n_tok, &pa, &why) != Err::ok) return false;
      pool.commit_append(std::move(pa));
      return true;
    };
    if (root_len && !append(root, root_len)) return fail(why);
    const int n = pick(1, 6);
    std::vector<int64_t> seqs;
    std::vector<int32_t> n_new;
    for (int i = 0; i < n; ++i) {
      int64_t c;
      if (pool.fork(root, &c, &why) != Err::ok) return fail(why);
      const int own = pick(0, 3) == 0 ? 0 : pick(1, 200);
      if (own && !append(c, own)) return fail(why);
      seqs.push_back(c);
      const SeqState* st = pool.find(c);
      n_new.push_back(pick(0, 2) == 0 ? st->len : std::min(st->len, own + pick(0, 5)));
    }
    Plan plan;
    if (plan_prefill(pool, seqs.data(), n, n_new.data(), cfg, &plan, &why) != Err::ok) return fail(why);
    ++plans;
    const int32_t G = sh.num_q_heads / sh.num_kv_heads, B = sh.block_size;
    std::vector<int32_t> q_seq, q_pos, blk_base(n, -1);
    int32_t base = 0;
    for (int i = 0; i < n; ++i) {
      const SeqState* st = pool.find(seqs[i]);
      if (n_new[i] > 0) {
        blk_base[i] = base;
        base += static_cast<int32_t>(st->table.size());
      }
      for (int j = 0; j < n_new[i]; ++j) {
        q_seq.push_back(i);
        q_pos.push_back(st->len - n_new[i] + j);
      }
    }
    const size_t nq = q_seq.size();
    std::vector<std::vector<int>> seen(nq);
    for (size_t q = 0; q < nq; ++q) seen[q].assign(q_pos[q] + 1, 0);
    const int32_t mrows = mfma_item_rows(plan.mfma_row_tiles, plan.mfma_waves);
    for (const auto* items : {&plan.mfma, &plan.valu}) {
      const bool is_mfma = items == &plan.mfma;
      for (const WorkItem& it : *items) {
        if (it.n_tok < 1 || it.n_grp < 1) return fail("empty item");
        if (it.n_grp * G > (is_mfma ? mrows : 8)) return fail("too many rows");
        if (!is_mfma && it.n_tok > 512) return fail("VALU item too long");
        if ((it.n_tok + B - 1) / B > 512) return fail("item spans too many blocks");
        for (int u = 0; u < it.n_grp; ++u) {
          const RowGroup& g = plan.groups[it.grp_off + u];
          const int32_t q = g.q_index;
          const int i = q_seq[q];
          const SeqState* st = pool.find(seqs[i]);
          const uint64_t anc = (static_cast<uint64_t>(g.anc_hi) << 32) | g.anc_lo;
          for (int32_t t = 0; t < it.n_tok; ++t) {
            const int32_t pos = (it.blk_off - blk_base[i]) * B + t;
            if (plan.blocks[it.blk_off + t / B] != st->table[pos / B]) return fail("wrong block");
            bool vis = true;
            if (t >= it.tail_start) {
              const int32_t sh_amt = it.tail_node0 + t - it.tail_start;
              if (sh_amt < 0 || sh_amt > 63) return fail("mask shift out of range");
              vis = (anc >> sh_amt) & 1;
            }
            if (!vis) continue;
            if (pos > q_pos[q]) return fail("a key after the query is visible");
            ++seen[q][pos];
          }
        }
      }
    }
    for (size_t q = 0; q < nq; ++q)
      for (int32_t p = 0; p <= q_pos[q]; ++p)
        if (seen[q][p] != 1)
          return fail("query " + std::to_string(q) + " sees key " + std::to_string(p) + " " +
                      std::to_string(seen[q][p]) + " times");
    // merge bookkeeping: single-part queries write directly, others have a merge row
    std::vector<int> parts(nq, 0);
    for (const auto* items : {&plan.mfma, &plan.valu})
      for (const WorkItem& it : *items)
        for (int u = 0; u < it.n_grp; ++u) ++parts[plan.groups[it.grp_off + u].q_index];
    for (const MergeRow& m : plan.merges)
      if (m.n_parts != parts[m.q_index]) return fail("merge row part count");
    size_t multi = 0;
    for (size_t q = 0; q < nq; ++q) multi += parts[q] > 1;
    if (multi != plan.merges.size()) return fail("merge rows");
  }
  std::printf("ok %d plans\n", plans);
  return 0;
}
