// Random prefix-cache traffic over a host pool, for sanitizer builds of the
// host sources: requests draw prompts from a few shared stems, match the
// cache, append what it misses, insert, release, evict under pressure, and
// sometimes fork or free; the pool's refcounts must balance at the end
// (every block back on the free list once the cache is emptied).
// Prints "ok <requests>" or "FAIL <what>".
#include <cstdio>
#include <cstdlib>
#include <random>
#include <string>
#include <vector>

#include "host/pool.hpp"
#include "host/radix.hpp"

using namespace pkv;

int main(int argc, char** argv) {
  const uint32_t seed = argc > 1 ? static_cast<uint32_t>(std::atoi(argv[1])) : 1;
  const int rounds = argc > 2 ? std::atoi(argv[2]) : 400;
  std::mt19937 rng(seed);
  const int32_t B = 1 << (rng() % 4);   // 1, 2, 4 or 8 tokens per block
  const Shape sh{96, B, 1, 4, 2, 8};
  BlockPool pool(sh, nullptr);
  RadixCache cache(&pool);
  std::vector<std::vector<int32_t>> stems(4);
  for (auto& s : stems) {
    s.resize(20 + rng() % 40);
    for (auto& t : s) t = static_cast<int32_t>(rng() % 50);
  }
  std::string why;
  std::vector<int64_t> live;
  for (int r = 0; r < rounds; ++r) {
    std::vector<int32_t> prompt = stems[rng() % stems.size()];
    prompt.resize(prompt.size() - rng() % 10);
    const int extra = static_cast<int>(rng() % 24);
    for (int i = 0; i < extra; ++i) prompt.push_back(static_cast<int32_t>(rng() % 50));
    int64_t seq = -1;
    int32_t hit = 0;
    if (cache.match(prompt.data(), static_cast<int32_t>(prompt.size()), &seq, &hit, &why) != Err::ok) {
      std::printf("FAIL match: %s\n", why.c_str());
      return 1;
    }
    const int32_t miss = static_cast<int32_t>(prompt.size()) - hit;
    if (miss > 0) {
      PendingAppend pa;
      Err e = pool.prepare_append(&seq, 1, miss, &pa, &why);
      if (e == Err::oom) {
        cache.evict(16);
        e = pool.prepare_append(&seq, 1, miss, &pa, &why);
      }
      if (e == Err::oom) {   // still full: give this request up
        if (cache.release(seq, &why) != Err::ok || pool.release(seq, &why) != Err::ok) {
          std::printf("FAIL give up: %s\n", why.c_str());
          return 1;
        }
        continue;
      }
      if (e != Err::ok) {
        std::printf("FAIL append: %s\n", why.c_str());
        return 1;
      }
      pool.commit_append(std::move(pa));
    }
    if (cache.insert(seq, prompt.data(), static_cast<int32_t>(prompt.size()), &why) != Err::ok) {
      std::printf("FAIL insert: %s\n", why.c_str());
      return 1;
    }
    if (rng() % 3 == 0) {
      int64_t child;
      if (pool.fork(seq, &child, &why) == Err::ok) live.push_back(child);
    }
    if (cache.release(seq, &why) != Err::ok || pool.release(seq, &why) != Err::ok) {
      std::printf("FAIL release: %s\n", why.c_str());
      return 1;
    }
    if (!live.empty() && rng() % 2 == 0) {
      const size_t k = rng() % live.size();
      if (pool.release(live[k], &why) != Err::ok) {
        std::printf("FAIL free fork: %s\n", why.c_str());
        return 1;
      }
      live.erase(live.begin() + static_cast<long>(k));
    }
  }
  for (int64_t s : live)
    if (pool.release(s, &why) != Err::ok) {
      std::printf("FAIL final free: %s\n", why.c_str());
      return 1;
    }
  if (!cache.evict(sh.num_blocks)) {
    std::printf("FAIL evict: a node still locked after every release\n");
    return 1;
  }
  if (cache.cached_blocks() != 0 || static_cast<int32_t>(pool.free_list().size()) != sh.num_blocks) {
    std::printf("FAIL leak: %d cached, %d free of %d\n", cache.cached_blocks(), static_cast<int32_t>(pool.free_list().size()), sh.num_blocks);
    return 1;
  }
  std::printf("ok %d\n", rounds);
  return 0;
}
