#include "pool.hpp"

#include <unordered_set>

namespace pkv {

bool valid_shape(const Shape& s, std::string* why) {
  auto fail = [&](const char* m) {
    if (why) *why = m;
    return false;
  };
  if (s.num_blocks < 1) return fail("num_blocks must be >= 1");
  if (s.block_size < 1 || s.block_size > 128 || (s.block_size & (s.block_size - 1)))
    return fail("block_size must be a power of two in 1..128");
  if (s.num_layers < 1) return fail("num_layers must be >= 1");
  if (s.num_kv_heads < 1 || s.num_q_heads < 1 || s.num_q_heads % s.num_kv_heads)
    return fail("num_q_heads must be a positive multiple of num_kv_heads");
  if (s.head_dim < 1) return fail("head_dim must be >= 1");
  if (static_cast<int64_t>(s.num_blocks) * s.block_size > INT32_MAX)
    return fail("num_blocks * block_size must fit in int32");
  return true;
}

BlockPool::BlockPool(const Shape& s, const int32_t* free_order)
    : shape_(s), rc_(s.num_blocks, 0) {
  while ((1 << log2b_) < s.block_size) ++log2b_;
  for (int32_t i = 0; i < s.num_blocks; ++i)
    fifo_.push_back(free_order ? free_order[i] : i);
}

int64_t BlockPool::allocate() {
  int64_t id = next_id_++;
  SeqState s;
  s.epoch = ++epochs_;
  seqs_.emplace(id, std::move(s));
  ++version_;
  return id;
}

Err BlockPool::adopt(const int32_t* blocks, int32_t n_blocks, int32_t len, int64_t* seq,
                     std::string* why) {
  const int32_t B = shape_.block_size;
  if (n_blocks < 0 || (n_blocks > 0 && !blocks) ||
      (n_blocks == 0 ? len != 0 : (len <= (n_blocks - 1) * B || len > n_blocks * B))) {
    *why = "adopt: length does not match the block count";
    return Err::arg;
  }
  for (int32_t i = 0; i < n_blocks; ++i)
    if (blocks[i] < 0 || blocks[i] >= shape_.num_blocks || rc_[blocks[i]] < 1) {
      *why = "adopt: block " + std::to_string(blocks[i]) + " is not held";
      return Err::arg;
    }
  SeqState s;
  s.table.assign(blocks, blocks + n_blocks);
  s.len = len;
  s.epoch = ++epochs_;
  for (int32_t b : s.table) ++rc_[b];
  const int64_t id = next_id_++;
  seqs_.emplace(id, std::move(s));
  *seq = id;
  ++version_;
  return Err::ok;
}

void BlockPool::retain(int32_t block) {
  ++rc_[block];
  ++version_;
}

void BlockPool::drop(int32_t block) {
  if (--rc_[block] == 0) fifo_.push_back(block);
  ++version_;
}

const SeqState* BlockPool::find(int64_t seq) const {
  auto it = seqs_.find(seq);
  return it == seqs_.end() ? nullptr : &it->second;
}

Err BlockPool::fork(int64_t parent, int64_t* child, std::string* why) {
  auto it = seqs_.find(parent);
  if (it == seqs_.end()) {
    *why = "seq_fork: unknown parent sequence " + std::to_string(parent);
    return Err::seq;
  }
  SeqState copy = it->second;  // table pointers only; no K/V moves
  copy.epoch = ++epochs_;
  for (int32_t b : copy.table) ++rc_[b];
  int64_t id = next_id_++;
  seqs_.emplace(id, std::move(copy));
  *child = id;
  ++version_;
  return Err::ok;
}

Err BlockPool::release(int64_t seq, std::string* why) {
  auto it = seqs_.find(seq);
  if (it == seqs_.end()) {
    *why = "seq_free: unknown sequence " + std::to_string(seq);
    return Err::seq;
  }
  for (int32_t b : it->second.table) {
    if (--rc_[b] == 0) fifo_.push_back(b);
  }
  seqs_.erase(it);
  ++version_;
  return Err::ok;
}

Err BlockPool::prepare_append(const int64_t* seqs, int32_t n_seqs, int32_t n_tok,
                              PendingAppend* out, std::string* why) const {
  if (n_seqs < 0 || n_tok < 0) {
    *why = "kv_append: negative count";
    return Err::arg;
  }
  if (n_seqs > 0 && !seqs) {
    *why = "kv_append: seqs is NULL";
    return Err::arg;
  }
  const int32_t B = shape_.block_size;
  std::vector<const SeqState*> st(n_seqs);
  {
    std::unordered_set<int64_t> seen;
    for (int32_t i = 0; i < n_seqs; ++i) {
      auto it = seqs_.find(seqs[i]);
      if (it == seqs_.end()) {
        *why = "kv_append: unknown sequence " + std::to_string(seqs[i]);
        return Err::seq;
      }
      if (!seen.insert(seqs[i]).second) {
        *why = "kv_append: sequence " + std::to_string(seqs[i]) + " appears twice";
        return Err::arg;
      }
      if (static_cast<int64_t>(it->second.len) + n_tok > INT32_MAX / 2) {
        *why = "kv_append: sequence length would overflow";
        return Err::arg;
      }
      st[i] = &it->second;
    }
  }
  // Simulate on copies.  Touched refcounts live in a side map; blocks come
  // from the free-list head in order.
  std::unordered_map<int32_t, int32_t> rcm;
  auto rc_of = [&](int32_t b) {
    auto it = rcm.find(b);
    return it == rcm.end() ? rc_[b] : it->second;
  };
  size_t taken = 0;
  out->result.slots.assign(static_cast<size_t>(n_seqs) * n_tok, 0);
  out->result.cow.clear();
  out->states.clear();
  out->states.reserve(n_seqs);
  for (int32_t i = 0; i < n_seqs && n_tok > 0; ++i) {
    SeqState s = *st[i];
    for (int32_t j = 0; j < n_tok; ++j) {
      const int32_t off = s.len % B;
      if (off == 0) {
        if (taken >= fifo_.size()) {
          *why = "kv_append: pool exhausted (" + std::to_string(fifo_.size()) + " free blocks)";
          return Err::oom;
        }
        const int32_t b = fifo_[taken++];
        rcm[b] = 1;
        s.table.push_back(b);
        s.epoch = 0;   // a new one at commit
      } else if (rc_of(s.table.back()) > 1) {
        if (taken >= fifo_.size()) {
          *why = "kv_append: pool exhausted (" + std::to_string(fifo_.size()) + " free blocks)";
          return Err::oom;
        }
        const int32_t src = s.table.back();
        const int32_t dst = fifo_[taken++];
        rcm[dst] = 1;
        rcm[src] = rc_of(src) - 1;
        s.table.back() = dst;
        s.epoch = 0;
        out->result.cow.push_back(CowCopy{src, dst, off});
      }
      out->result.slots[static_cast<size_t>(i) * n_tok + j] = s.table[s.len / B] * B + off;
      ++s.len;
    }
    out->states.emplace_back(seqs[i], std::move(s));
  }
  out->refcounts.assign(rcm.begin(), rcm.end());
  out->taken = taken;
  out->version = version_;
  return Err::ok;
}

void BlockPool::commit_append(PendingAppend&& pa) {
  for (size_t k = 0; k < pa.taken; ++k) fifo_.pop_front();
  for (const auto& br : pa.refcounts) rc_[br.first] = br.second;
  for (auto& ss : pa.states) {
    if (ss.second.epoch == 0) ss.second.epoch = ++epochs_;
    seqs_[ss.first] = std::move(ss.second);
  }
  if (!pa.states.empty()) ++version_;
  last_append_ = std::move(pa.result);
}

Err BlockPool::prepare_commit(const int64_t* seqs, int32_t n_seqs, int32_t n_nodes,
                              const int32_t* parent, const int32_t* path_len, const int32_t* paths,
                              PendingCommit* out, std::string* why) const {
  if (n_seqs < 0 || (n_seqs > 0 && (!seqs || !parent || !path_len || !paths))) {
    *why = "kv_tree_commit: bad arguments";
    return Err::arg;
  }
  if (n_seqs > 0 && (n_nodes < 1 || n_nodes > 64)) {
    *why = "kv_tree_commit: n_nodes must be in 1..64";
    return Err::arg;
  }
  const int32_t B = shape_.block_size;
  std::vector<const SeqState*> st(n_seqs);
  {
    std::unordered_set<int64_t> seen;
    for (int32_t i = 0; i < n_seqs; ++i) {
      auto it = seqs_.find(seqs[i]);
      if (it == seqs_.end()) {
        *why = "kv_tree_commit: unknown sequence " + std::to_string(seqs[i]);
        return Err::seq;
      }
      if (!seen.insert(seqs[i]).second) {
        *why = "kv_tree_commit: sequence " + std::to_string(seqs[i]) + " appears twice";
        return Err::arg;
      }
      if (it->second.len < n_nodes) {
        *why = "kv_tree_commit: sequence " + std::to_string(seqs[i]) + " is shorter than its tree";
        return Err::arg;
      }
      const int32_t* par = parent + static_cast<size_t>(i) * n_nodes;
      bool tree = par[0] == -1;
      for (int32_t j = 1; j < n_nodes && tree; ++j) tree = par[j] >= 0 && par[j] < j;
      const int32_t np = path_len[i];
      const int32_t* pa = paths + static_cast<size_t>(i) * n_nodes;
      bool ok = tree && np >= 0 && np <= n_nodes && (np == 0 || pa[0] == 0);
      for (int32_t k = 1; k < np && ok; ++k) ok = pa[k] > 0 && pa[k] < n_nodes && par[pa[k]] == pa[k - 1];
      if (!ok) {
        *why = "kv_tree_commit: sequence " + std::to_string(seqs[i]) +
               ": parent[] is not a tree in node order or the path does not run from the root "
               "along parent links";
        return Err::arg;
      }
      st[i] = &it->second;
    }
  }
  std::unordered_map<int32_t, int32_t> rcm;
  auto rc_of = [&](int32_t b) {
    auto it = rcm.find(b);
    return it == rcm.end() ? rc_[b] : it->second;
  };
  out->states.clear();
  out->pushed.clear();
  out->cow.clear();
  out->move_src.clear();
  out->move_dst.clear();
  out->seq_cow.assign(1, 0);
  out->seq_move.assign(1, 0);
  out->taken = 0;
  out->conflict = false;
  // old tree block -> the sequence reading it (-2: more than one)
  std::unordered_map<int32_t, int32_t> reader;
  std::vector<std::pair<int32_t, int32_t>> in_place;   // (block, sequence) written without a copy
  for (int32_t i = 0; i < n_seqs; ++i) {
    SeqState s = *st[i];
    const int32_t np = path_len[i];
    const int32_t* pa = paths + static_cast<size_t>(i) * n_nodes;
    const int32_t ctx = s.len - n_nodes;
    const int32_t new_len = ctx + np;
    const int32_t keep = (new_len + B - 1) / B;
    for (size_t b = keep; b < s.table.size(); ++b) {
      const int32_t blk = s.table[b];
      const int32_t r = rc_of(blk) - 1;
      rcm[blk] = r;
      if (r == 0) out->pushed.push_back(blk);
    }
    const std::vector<int32_t> old = s.table;
    s.table.resize(keep);
    int32_t last_written = -1;
    for (int32_t k = 0; k < np; ++k) {
      if (pa[k] == k) continue;
      const int32_t bi = (ctx + k) / B;
      if (bi != last_written) {
        last_written = bi;
        if (rc_of(s.table[bi]) > 1) {
          // copies take blocks that were free before the call, never one this
          // call releases (its old tokens may still be read by a move)
          if (out->taken >= fifo_.size()) {
            *why = "kv_tree_commit: pool exhausted (copy-on-write of a shared tree block)";
            return Err::oom;
          }
          const int32_t dst = fifo_[out->taken];
          ++out->taken;
          const int32_t src = s.table[bi];
          rcm[dst] = 1;
          rcm[src] = rc_of(src) - 1;
          s.table[bi] = dst;
          out->cow.push_back(CowCopy{src, dst, std::min(B, new_len - bi * B)});
        } else {
          in_place.emplace_back(s.table[bi], i);
        }
      }
      const int32_t sp = ctx + pa[k];
      const int32_t sb = old[sp / B];
      auto rd = reader.emplace(sb, i);
      if (!rd.second && rd.first->second != i) rd.first->second = -2;
      out->move_src.push_back(sb * B + sp % B);
      out->move_dst.push_back(s.table[bi] * B + (ctx + k) % B);
    }
    s.len = new_len;
    s.epoch = 0;
    out->states.emplace_back(seqs[i], std::move(s));
    out->seq_cow.push_back(static_cast<int32_t>(out->cow.size()));
    out->seq_move.push_back(static_cast<int32_t>(out->move_src.size()));
  }
  // every sequence's moves read its old blocks; a block written in place by
  // one sequence and read by another needs the sequences in order
  for (const auto& w : in_place) {
    auto it = reader.find(w.first);
    if (it != reader.end() && it->second != w.second) out->conflict = true;   // -2 included
  }
  out->refcounts.assign(rcm.begin(), rcm.end());
  out->version = version_;
  return Err::ok;
}

void BlockPool::commit_commit(PendingCommit&& pc) {
  for (int32_t b : pc.pushed) fifo_.push_back(b);
  for (size_t k = 0; k < pc.taken; ++k) fifo_.pop_front();
  for (const auto& br : pc.refcounts) rc_[br.first] = br.second;
  for (auto& ss : pc.states) {
    ss.second.epoch = ++epochs_;
    seqs_[ss.first] = std::move(ss.second);
  }
  if (!pc.states.empty()) ++version_;
}

}  // namespace pkv
