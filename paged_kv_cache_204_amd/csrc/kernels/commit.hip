// kv_tree_commit device work: after a draft tree is verified, the accepted
// path's K/V move to the positions right after the context and the rest is
// dropped (CAST page: the target keeps the draft tokens it accepts).
//
// One thread owns one column of the pool -- (layer, K or V, kv head,
// 16-byte chunk of head_dim) -- for one sequence and does that sequence's
// work on it in order: first the copy-on-write copies (slots [0, n) of a
// shared block into its fresh copy), then the token moves in path order.
// Move k reads old position ctx + path[k] >= ctx + k and writes ctx + k;
// earlier moves wrote only positions below ctx + k, so no move reads a slot
// an earlier one wrote.  That lets a thread load eight sources before it
// stores them.  Copies write only blocks that were free before the call,
// which no move reads.  Sequences run side by side unless one writes in
// place a block another reads (the host then launches them one by one).
#include "../kernels.hpp"
#include "common.hpp"

namespace pkv {
namespace {

__global__ __launch_bounds__(256) void commit_kernel(CommitParams p) {
  const int32_t cpr = p.D / 8;
  const int32_t cols = p.L * 2 * p.Hkv * cpr;
  const int32_t col = static_cast<int32_t>(blockIdx.x) * 256 + static_cast<int32_t>(threadIdx.x);
  if (col >= cols) return;
  const int32_t seq = p.seq0 + static_cast<int32_t>(blockIdx.y);
  const int32_t c = col % cpr;
  int32_t r = col / cpr;
  const int32_t h = r % p.Hkv;
  r /= p.Hkv;
  const int32_t kv = r & 1;
  const int32_t l = r >> 1;
  uint16_t* pool = kv ? p.v_pool : p.k_pool;
  const int64_t head_tile = static_cast<int64_t>(p.B) * p.D;
  const int64_t block_elems = head_tile * p.Hkv;
  uint16_t* col_base = pool + static_cast<int64_t>(l) * block_elems * p.N + h * head_tile + c * 8;
  auto at = [&](int32_t blk, int32_t off) {
    return reinterpret_cast<uint4*>(col_base + blk * block_elems + static_cast<int64_t>(off) * p.D);
  };
  for (int32_t i = p.seq_cow[seq]; i < p.seq_cow[seq + 1]; ++i) {
    const int32_t src = p.cow[3 * i + 0];
    const int32_t dst = p.cow[3 * i + 1];
    const int32_t n = p.cow[3 * i + 2];
    for (int32_t o = 0; o < n; ++o) *at(dst, o) = *at(src, o);
  }
  const int32_t m0 = p.seq_move[seq], m1 = p.seq_move[seq + 1];
  for (int32_t k0 = m0; k0 < m1; k0 += 8) {
    uint4 v[8];
#pragma unroll
    for (int32_t j = 0; j < 8; ++j)
      if (k0 + j < m1) {
        const int32_t s = p.move_src[k0 + j];
        v[j] = *at(s >> p.log2B, s & (p.B - 1));
      }
#pragma unroll
    for (int32_t j = 0; j < 8; ++j)
      if (k0 + j < m1) {
        const int32_t d = p.move_dst[k0 + j];
        *at(d >> p.log2B, d & (p.B - 1)) = v[j];
      }
  }
}

}  // namespace

hipError_t launch_commit(const CommitParams& p, int32_t n_seqs, hipStream_t s) {
  const int64_t cols = static_cast<int64_t>(p.L) * 2 * p.Hkv * (p.D / 8);
  if (cols == 0 || n_seqs == 0) return hipSuccess;
  hipLaunchKernelGGL(commit_kernel, dim3(static_cast<uint32_t>((cols + 255) / 256), static_cast<uint32_t>(n_seqs)),
                     dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace pkv
