#include "radix.hpp"

#include <algorithm>

namespace pkv {

RadixCache::RadixCache(BlockPool* pool) : pool_(pool) {}

RadixCache::~RadixCache() {
  if (!pool_) return;
  // preorder, children in key order, each edge's blocks in order
  std::vector<RadixNode*> stack{&root_};
  while (!stack.empty()) {
    RadixNode* n = stack.back();
    stack.pop_back();
    for (int32_t b : n->blocks) pool_->drop(b);
    for (auto it = n->children.rbegin(); it != n->children.rend(); ++it) stack.push_back(it->second.get());
  }
}

Err RadixCache::match(const int32_t* tokens, int32_t n, int64_t* seq, int32_t* matched,
                      std::string* why) {
  if (n < 0 || (n > 0 && !tokens)) {
    *why = "radix_match: bad token array";
    return Err::arg;
  }
  const int32_t B = cpool().shape().block_size;
  std::vector<int32_t> blocks;
  std::vector<int32_t> key(B);
  RadixNode* cur = &root_;
  RadixNode* deepest = nullptr;
  int32_t reach = 0;
  int32_t pos = 0;
  while (pos + B <= n) {
    key.assign(tokens + pos, tokens + pos + B);
    auto it = cur->children.find(key);
    if (it == cur->children.end()) break;
    RadixNode* c = it->second.get();
    const int32_t nb = static_cast<int32_t>(c->blocks.size());
    int32_t m = 1;   // the key is the edge's first block
    while (m < nb && pos + (m + 1) * B <= n &&
           std::equal(tokens + pos + m * B, tokens + pos + (m + 1) * B, c->tokens.begin() + m * B))
      ++m;
    blocks.insert(blocks.end(), c->blocks.begin(), c->blocks.begin() + m);
    deepest = c;
    reach = m * B;
    pos += m * B;
    if (m < nb) break;   // the prompt leaves this edge part-way (split on a later insert)
    cur = c;
  }
  int64_t id;
  Err e = pool_->adopt(blocks.data(), static_cast<int32_t>(blocks.size()), pos, &id, why);
  if (e != Err::ok) return e;
  std::vector<RadixNode*> path;
  for (RadixNode* p = deepest; p && p != &root_; p = p->parent) path.push_back(p);
  for (auto it = path.rbegin(); it != path.rend(); ++it) {
    ++(*it)->lock;
    touch(*it);
  }
  matched_[id] = Held{deepest, reach};
  *seq = id;
  *matched = pos;
  return Err::ok;
}

RadixNode* RadixCache::split(RadixNode* child, int32_t keep) {
  const int32_t B = cpool().shape().block_size;
  RadixNode* parent = child->parent;
  auto mid = std::make_unique<RadixNode>();
  mid->tokens.assign(child->tokens.begin(), child->tokens.begin() + keep * B);
  mid->blocks.assign(child->blocks.begin(), child->blocks.begin() + keep);
  child->tokens.erase(child->tokens.begin(), child->tokens.begin() + keep * B);
  child->blocks.erase(child->blocks.begin(), child->blocks.begin() + keep);
  mid->parent = parent;
  // every match that locked the child ran through the common part too; the
  // ones that ended within it now end at the new parent
  mid->lock = child->lock;
  mid->last_access = child->last_access;
  for (auto& kv : matched_) {
    Held& h = kv.second;
    if (h.node != child) continue;
    if (h.reach <= keep * B) {
      h.node = mid.get();
      --child->lock;
    } else {
      h.reach -= keep * B;
    }
  }
  const std::vector<int32_t> key(mid->tokens.begin(), mid->tokens.begin() + B);
  std::unique_ptr<RadixNode> owned = std::move(parent->children[key]);
  RadixNode* m = mid.get();
  parent->children[key] = std::move(mid);
  child->parent = m;
  m->children[std::vector<int32_t>(child->tokens.begin(), child->tokens.begin() + B)] = std::move(owned);
  ++n_nodes_;
  return m;
}

Err RadixCache::insert(int64_t seq, const int32_t* tokens, int32_t n, std::string* why) {
  const SeqState* st = cpool().find(seq);
  if (!st) {
    *why = "radix_insert: unknown sequence " + std::to_string(seq);
    return Err::seq;
  }
  if (n < 0 || n > st->len || (n > 0 && !tokens)) {
    *why = "radix_insert: token count outside 0..len or NULL tokens";
    return Err::arg;
  }
  const int32_t B = cpool().shape().block_size;
  const int32_t nb_total = n / B;   // whole blocks only
  std::vector<int32_t> key(B);
  RadixNode* cur = &root_;
  int32_t bi = 0;
  while (bi < nb_total) {
    key.assign(tokens + bi * B, tokens + (bi + 1) * B);
    auto it = cur->children.find(key);
    if (it == cur->children.end()) {
      auto leaf = std::make_unique<RadixNode>();
      leaf->tokens.assign(tokens + bi * B, tokens + nb_total * B);
      leaf->blocks.assign(st->table.begin() + bi, st->table.begin() + nb_total);
      for (int32_t b : leaf->blocks) pool_->retain(b);
      leaf->parent = cur;
      touch(leaf.get());
      n_blocks_ += nb_total - bi;
      ++n_nodes_;
      cur->children[key] = std::move(leaf);
      break;
    }
    RadixNode* c = it->second.get();
    touch(c);
    const int32_t nb = static_cast<int32_t>(c->blocks.size());
    int32_t m = 1;
    while (m < nb && bi + m < nb_total &&
           std::equal(tokens + (bi + m) * B, tokens + (bi + m + 1) * B, c->tokens.begin() + m * B))
      ++m;
    if (m < nb) {
      if (bi + m == nb_total) break;   // the run ends inside this edge: already cached
      c = split(c, m);                 // diverges part-way: common blocks become the parent
    }
    bi += m;
    cur = c;
  }
  return Err::ok;
}

Err RadixCache::release(int64_t seq, std::string* why) {
  auto it = matched_.find(seq);
  if (it == matched_.end()) {
    *why = "radix_release: sequence " + std::to_string(seq) + " holds no match of this cache";
    return Err::seq;
  }
  for (RadixNode* p = it->second.node; p && p != &root_; p = p->parent) --p->lock;
  matched_.erase(it);
  return Err::ok;
}

bool RadixCache::evict(int32_t want_free) {
  while (static_cast<int64_t>(cpool().free_list().size()) < want_free) {
    RadixNode* best = nullptr;
    std::vector<RadixNode*> stack{&root_};
    while (!stack.empty()) {
      RadixNode* n = stack.back();
      stack.pop_back();
      if (n != &root_ && n->children.empty() && n->lock == 0 &&
          (!best || n->last_access < best->last_access))
        best = n;
      for (auto& kv : n->children) stack.push_back(kv.second.get());
    }
    if (!best) return false;   // every cached block sits under a live match
    for (int32_t b : best->blocks) pool_->drop(b);
    n_blocks_ -= static_cast<int32_t>(best->blocks.size());
    --n_nodes_;
    const int32_t B = cpool().shape().block_size;
    RadixNode* parent = best->parent;
    parent->children.erase(std::vector<int32_t>(best->tokens.begin(), best->tokens.begin() + B));
  }
  return true;
}

int32_t RadixCache::locked_nodes() const {
  int32_t k = 0;
  std::vector<const RadixNode*> stack{&root_};
  while (!stack.empty()) {
    const RadixNode* n = stack.back();
    stack.pop_back();
    if (n != &root_ && n->lock > 0) ++k;
    for (const auto& kv : n->children) stack.push_back(kv.second.get());
  }
  return k;
}

void RadixCache::dump(std::vector<int32_t>* out) const {
  out->clear();
  // preorder, children in key order
  std::vector<std::pair<const RadixNode*, int32_t>> stack;
  for (auto it = root_.children.rbegin(); it != root_.children.rend(); ++it)
    stack.emplace_back(it->second.get(), 1);
  while (!stack.empty()) {
    auto [n, depth] = stack.back();
    stack.pop_back();
    out->push_back(depth);
    out->push_back(static_cast<int32_t>(n->tokens.size()));
    out->push_back(n->lock);
    out->insert(out->end(), n->tokens.begin(), n->tokens.end());
    out->insert(out->end(), n->blocks.begin(), n->blocks.end());
    for (auto it = n->children.rbegin(); it != n->children.rend(); ++it)
      stack.emplace_back(it->second.get(), depth + 1);
  }
}

}  // namespace pkv
